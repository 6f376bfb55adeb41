"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU involved):

* the oracle (oracle/gdr_oracle.c), every route with every intermediate export, driven by
  tests/sanitize/oracle_driver.c;
* the host entry points (gated_delta_rule_70_amd/csrc/gdr_api.cpp) with the kernel
  launchers stubbed out (tests/sanitize/stub_launchers.cpp), every validation path driven by
  tests/sanitize/api_driver.c on fake device addresses that no call dereferences.

Sanitizers apply to host code only (the device pass of gdr_api.cpp is built without them).
Any sanitizer report aborts the program, which fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "gated_delta_rule_70_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = "/opt/rocm/bin/hipcc"
SAN_FLAGS = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", *SAN_FLAGS, os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "gdr_oracle.c"), "-lm", "-o", exe])
    res = _run([exe], env=ENV, timeout=300)
    assert "oracle sanitize ok" in res.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not available")
def test_host_entry_points_under_sanitizers(tmp_path):
    host_san = [f for flag in SAN_FLAGS for f in ("-Xarch_host", flag)]
    objs = []
    for src in (os.path.join(CSRC, "gdr_api.cpp"), os.path.join(SAN, "stub_launchers.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", *host_san, "-I", INCLUDE, "-I", CSRC,
              "-x", "hip", "-c", src, "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "api_driver.o")
    _run([CLANG, "-O1", "-g", "-std=c99", *SAN_FLAGS, "-I", INCLUDE, "-c", os.path.join(SAN, "api_driver.c"), "-o", drv])
    exe = str(tmp_path / "api_san")
    _run([HIPCC, "--offload-arch=gfx950", *host_san, drv, *objs, "-o", exe])
    res = _run([exe], env=ENV, timeout=300)
    assert "api sanitize ok" in res.stdout
