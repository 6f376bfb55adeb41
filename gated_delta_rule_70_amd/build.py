"""Build libgdr.so (HIP kernels for gfx950 + the C-ABI host entry points) in-tree.

Usage: ``python -m gated_delta_rule_70_amd.build`` (or ``build()`` from Python).  Each
translation unit is compiled by hipcc in parallel, then linked into
``gated_delta_rule_70_amd/libgdr.so``.  The library links against the HIP runtime by
SONAME (libamdhip64.so.7), so inside a process that already loaded PyTorch's bundled
runtime it binds to that same runtime and shares its streams and device pointers.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdr.so")

SOURCES = ["gdr_api.cpp", "decode.hip", "chunk_prep.hip", "chunk_prep_split.hip", "chunk_carry.hip",
           "chunk_carry_wide.hip", "tree_verify.hip", "varlen_plan.hip"]
ARCH = os.environ.get("GDR_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU forms are kept out of the device code (plain fp32 FMAs only).
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-but-set-variable"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgdr.so)")


def _compile(src: str) -> str:
    out = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    # the host pass does not know the gfx950 feature flag; that warning is expected
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in res.stderr.splitlines() if ln.strip() and noise not in ln]
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return out


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
