"""The C ABI of libgdr.so on the host: it loads, exports every declared symbol, sizes the
workspace, and rejects bad arguments before touching any GPU.

No test here launches a kernel.  Fake device addresses are used only on paths whose
validation fails on the host (the library runs every check before its first HIP call).
"""
import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_70_amd as gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

OK, ENULL, ESHAPE, EUNSUP, EALIGN, EALIAS, EWS, EHIP = range(8)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gdr.LIB_PATH):
        from gated_delta_rule_70_amd import build

        build.build(verbose=False)
    return gdr.lib()


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(gdr_\w+)\s*\(", src, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "gdr_abi_version", "gdr_chunk_carry", "gdr_chunk_prefill", "gdr_chunk_prefill_workspace_bytes",
        "gdr_chunk_prefill_noalloc", "gdr_chunk_prep", "gdr_decode_step", "gdr_forward",
        "gdr_fused_recurrent", "gdr_status_str", "gdr_tree_verify", "gdr_chunk_prefill_varlen",
        "gdr_chunk_prefill_varlen_workspace_bytes", "gdr_fused_recurrent_varlen"])


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", gdr.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)


def test_version_and_status_strings(L):
    assert L.gdr_abi_version() == gdr.ABI_VERSION
    texts = {L.gdr_status_str(s).decode() for s in range(9)}
    assert len(texts) == 9
    assert L.gdr_status_str(99).decode() == "unknown status"


# fake, well-separated, 256-byte-aligned device addresses (never dereferenced)
BASE = 1 << 40
SLOT = 1 << 32


def addr(i, off=0):
    return ctypes.c_void_p(BASE + i * SLOT + off)


def dims(**kw):
    d = dict(B=2, T=5, HK=2, HV=4, dk=64, dv=32, chunk=16, qkv_dtype=0)
    d.update(kw)
    return gdr.Dims(**d)


def prefill(L, d, ws_bytes=None, entry="gdr_chunk_prefill", **ptrs):
    p = {n: addr(i) for i, n in enumerate(["q", "k", "v", "g", "beta", "h0", "o", "ht", "ws"])}
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = L.gdr_chunk_prefill_workspace_bytes(ctypes.byref(d)) if d is not None else 0
    return getattr(L, entry)(None if d is None else ctypes.byref(d), p["q"], p["k"], p["v"], p["g"],
                               p["beta"], p["h0"], p["o"], p["ht"], p["ws"], ctypes.c_size_t(ws_bytes),
                               None)


def decode(L, d, entry="gdr_decode_step", **ptrs):
    p = {n: addr(i) for i, n in enumerate(["q", "k", "v", "g", "beta", "h0", "o", "ht"])}
    p.update(ptrs)
    return getattr(L, entry)(None if d is None else ctypes.byref(d), p["q"], p["k"], p["v"], p["g"],
                             p["beta"], p["h0"], p["o"], p["ht"], None)


def test_null_arguments(L):
    assert prefill(L, None) == ENULL
    assert decode(L, None) == ENULL
    for name in ("q", "k", "v", "g", "beta", "o"):
        assert prefill(L, dims(), **{name: None}) == ENULL, name
        assert decode(L, dims(T=1), **{name: None}) == ENULL, name


@pytest.mark.parametrize("kw", [dict(B=0), dict(T=0), dict(HK=0), dict(HV=0), dict(HK=3, HV=4),
                                dict(B=-1), dict(T=1 << 30, B=1 << 10)])
def test_bad_shapes(L, kw):
    assert prefill(L, dims(**kw)) == ESHAPE


def test_decode_requires_one_token(L):
    assert decode(L, dims(T=2)) == ESHAPE


def test_fused_recurrent_validates_like_decode_for_any_T(L):
    rec = dict(entry="gdr_fused_recurrent")
    assert decode(L, None, **rec) == ENULL
    for name in ("q", "k", "v", "g", "beta", "o"):
        assert decode(L, dims(T=7), **rec, **{name: None}) == ENULL, name
    assert decode(L, dims(T=0), **rec) == ESHAPE
    assert decode(L, dims(HK=3, HV=4), **rec) == ESHAPE
    assert decode(L, dims(dk=48), **rec) == EUNSUP
    assert decode(L, dims(qkv_dtype=2), **rec) == EUNSUP
    # the chunk length is ignored: an unsupported one gets as far as the alignment check
    assert decode(L, dims(T=7, chunk=8), q=addr(0, 8), **rec) == EALIGN
    assert decode(L, dims(T=7), q=addr(0, 8), **rec) == EALIGN
    assert decode(L, dims(T=7), o=addr(0, 256), **rec) == EALIAS
    assert decode(L, dims(T=7), ht=addr(5, 256), **rec) == EALIAS


@pytest.mark.parametrize("kw", [dict(dk=48), dict(dv=256), dict(dk=16), dict(chunk=8),
                                dict(chunk=128), dict(qkv_dtype=2)])
def test_unsupported(L, kw):
    assert prefill(L, dims(**kw)) == EUNSUP


def test_misaligned_pointers(L):
    for name in ("q", "k", "v", "g", "beta", "h0", "o", "ht"):
        assert prefill(L, dims(), **{name: addr(9, 4)}) == EALIGN, name


def test_aliasing(L):
    d = dims()
    assert prefill(L, d, o=addr(0, 256)) == EALIAS           # o inside q
    assert prefill(L, d, ht=addr(3, 0)) == EALIAS            # ht over g
    assert prefill(L, d, ht=addr(5, 256)) == EALIAS          # ht partially over h0
    assert prefill(L, d, o=addr(7, 0)) == EALIAS             # o over ht
    assert prefill(L, d, ws=addr(6, 0)) == EALIAS            # workspace over o


@pytest.mark.parametrize("entry", ["gdr_chunk_prep", "gdr_chunk_carry"])
def test_stage_entries_validate_like_prefill(L, entry):
    assert prefill(L, None, entry=entry) == ENULL
    assert prefill(L, dims(B=0), entry=entry) == ESHAPE
    assert prefill(L, dims(dk=48), entry=entry) == EUNSUP
    assert prefill(L, dims(), entry=entry, q=addr(0, 8)) == EALIGN
    assert prefill(L, dims(), entry=entry, o=addr(0, 256)) == EALIAS
    assert prefill(L, dims(), entry=entry, ws_bytes=1) == EWS


def test_forward_routes_by_length(L):
    # short calls take the recurrence (no workspace needed), longer ones the chunked path
    # (which checks its workspace); both stop at validation here
    assert prefill(L, dims(T=8), entry="gdr_forward", q=addr(0, 8), ws=None, ws_bytes=0) == EALIGN
    assert prefill(L, dims(T=9), entry="gdr_forward", ws=None, ws_bytes=0) == EWS
    assert prefill(L, dims(T=9, chunk=8), entry="gdr_forward") == EUNSUP
    assert prefill(L, dims(T=8, chunk=8), entry="gdr_forward", q=addr(0, 8)) == EALIGN
    assert prefill(L, None, entry="gdr_forward") == ENULL


def tree(L, d, parent=addr(10), **ptrs):
    p = {n: addr(i) for i, n in enumerate(["q", "k", "v", "g", "beta", "h0", "o"])}
    p.update(ptrs)
    return L.gdr_tree_verify(None if d is None else ctypes.byref(d), parent, p["q"], p["k"], p["v"],
                             p["g"], p["beta"], p["h0"], p["o"], None)


def test_tree_verify_checks(L):
    assert tree(L, dims(T=9), parent=None) == ENULL
    assert tree(L, None) == ENULL
    assert tree(L, dims(T=9), q=None) == ENULL
    assert tree(L, dims(T=65)) == EUNSUP                        # at most 64 nodes
    assert tree(L, dims(T=9, dk=48)) == EUNSUP
    assert tree(L, dims(T=9), parent=addr(10, 2)) == EALIGN      # int32 entries
    assert tree(L, dims(T=9), q=addr(0, 8)) == EALIGN
    assert tree(L, dims(T=9), o=addr(10, 0)) == EALIAS           # o over parent
    assert tree(L, dims(T=9), o=addr(0, 256)) == EALIAS          # o inside q


def test_workspace_checks(L):
    d = dims()
    need = L.gdr_chunk_prefill_workspace_bytes(ctypes.byref(d))
    assert need > 0 and need % 256 == 0
    assert prefill(L, d, ws_bytes=need - 1) == EWS
    assert prefill(L, d, ws=None) == EWS
    assert prefill(L, d, ws=addr(8, 16)) == EWS


def test_31_bit_offset_limit(L):
    # One launch takes T rows per batch element while (T + chunk) * HV * max(dk, dv) * 4 <
    # 2^31: up to T = 131007 at HV=32, 128x128, chunk 64.  Longer dense prefills run as a
    # chain of windows of W = 130944 rows (the largest multiple of the chunk that fits); the
    # stage entry points and packed batches refuse them.
    d = dict(B=1, HK=16, HV=32, dk=128, dv=128, chunk=64)
    for entry in ("gdr_chunk_prep", "gdr_chunk_carry"):
        assert prefill(L, dims(T=131008, **d), entry=entry) == ESHAPE
        assert prefill(L, dims(T=131007, **d), entry=entry, ws_bytes=1) == EWS  # within the limit
    assert varlen_call(L, dims(T=131008, **d)) == ESHAPE
    assert prefill(L, dims(T=131008, **d), ws_bytes=1) == EWS  # chained: passes, then needs workspace
    one = L.gdr_chunk_prefill_workspace_bytes(ctypes.byref(dims(T=131007, **d)))
    assert one >= _records(1, 131007, 32, 128, 64)  # one launch: every record of the call


def test_windowed_workspace(L):
    """A chained prefill needs one window's records and carry scratch (the window's own carry
    plan), rounded to 256 bytes, plus one head group's state; independent of T and B."""
    d = dict(HK=16, HV=32, dk=128, dv=128, chunk=64)
    W = 130944
    one = L.gdr_chunk_prefill_workspace_bytes(ctypes.byref(dims(B=1, T=W, **d)))
    for B, T in ((1, 131008), (1, 10 * W + 5), (3, 2 * W)):
        got = L.gdr_chunk_prefill_workspace_bytes(ctypes.byref(dims(B=B, T=T, **d)))
        assert got == (one + 255) // 256 * 256 + 32 * 128 * 128 * 4, (B, T)


@pytest.mark.skipif("_gpu_visible()", reason="valid fake pointers would reach a real GPU")
def test_windowed_prefill_reaches_the_runtime_without_a_gpu(L):
    # tensors of several GiB: fake addresses 256 GiB apart so that none overlaps another
    far = {n: ctypes.c_void_p((1 << 44) + i * (1 << 38))
           for i, n in enumerate(["q", "k", "v", "g", "beta", "h0", "o", "ht", "ws"])}
    d = dict(B=2, T=300000, HK=16, HV=32, dk=128, dv=128, chunk=64)
    assert prefill(L, dims(**d), **far) == EHIP
    assert prefill(L, dims(**d), **dict(far, ht=None)) == EHIP


def test_workspace_size_formula(L):
    # one record per (batch, value head, chunk): fp16 operand fragments of 1 KiB each,
    # plus one 1 KiB block for the dk fp32 decay totals
    for (dk, C) in [(32, 16), (64, 32), (128, 64), (128, 16)]:
        d = dims(dk=dk, chunk=C, T=100)
        nb, nqs, kc, dkt = C // 16, (C + 31) // 32, dk // 32, dk // 16
        nfrag = 2 * nb * kc + dkt * nqs + 2 * nb * nqs  # Qt, -W, Kb, Tb, P
        rec = (nfrag + 1) * 1024
        nchunk = -(-100 // C)
        assert L.gdr_chunk_prefill_workspace_bytes(ctypes.byref(d)) == 2 * 4 * nchunk * rec
    assert L.gdr_chunk_prefill_workspace_bytes(ctypes.byref(dims(dk=48))) == 0
    assert L.gdr_chunk_prefill_workspace_bytes(None) == 0


def _records(B, T, HV, dk, C):
    nb, nqs, kc, dkt = C // 16, (C + 31) // 32, dk // 32, dk // 16
    return B * HV * (-(-T // C)) * ((2 * nb * kc + dkt * nqs + 2 * nb * nqs + 1) * 1024)


def test_workspace_carry_segments(L):
    """The segmented carry's extra workspace: with at most 128 (batch, head) pairs whose
    16-column tiles fit 256 workgroups and enough chunks for 256 / heads segments of >= 16
    chunks each, every segment but the last
    keeps an fp32 [S_loc | M] summary (2 dk x dk matrices) and every segment a start state
    (dk x dv); otherwise the workspace is the chunk records alone."""
    def ws(**kw):
        return L.gdr_chunk_prefill_workspace_bytes(ctypes.byref(dims(**kw)))
    # 2 heads, 2048 chunks of 16: 128 segments
    kw = dict(B=1, HK=1, HV=2, dk=128, dv=128, chunk=16, T=32768)
    nseg, mat = 128, 128 * 128 * 4
    assert ws(**kw) == _records(1, 32768, 2, 128, 16) + 2 * (nseg - 1) * 2 * mat + 2 * nseg * mat
    # 32 heads, 512 chunks of 64: 8 segments
    kw = dict(B=1, HK=16, HV=32, dk=128, dv=128, chunk=64, T=32768)
    assert ws(**kw) == _records(1, 32768, 32, 128, 64) + 32 * 7 * 2 * mat + 32 * 8 * mat
    # 32 heads, 65 chunks: too few for 8 segments of 16 -> column-split carry, records only
    kw = dict(B=1, HK=16, HV=32, dk=128, dv=128, chunk=64, T=4097)
    assert ws(**kw) == _records(1, 4097, 32, 128, 64)
    # 64 heads (512 tiles): column split with 2 tiles per workgroup, records only; the same
    # heads at dv = 64 (256 tiles) take 4 segments
    kw = dict(B=2, HK=16, HV=32, dk=128, dv=128, chunk=64, T=4097)
    assert ws(**kw) == _records(2, 4097, 32, 128, 64)
    kw = dict(B=2, HK=16, HV=32, dk=64, dv=64, chunk=64, T=4100)
    m64 = 64 * 64 * 4
    assert ws(**kw) == _records(2, 4100, 32, 64, 64) + 64 * 3 * 2 * m64 + 64 * 4 * m64
    # 256 heads: whole-head carry with a single segment, records only
    kw = dict(B=8, HK=16, HV=32, dk=128, dv=128, chunk=64, T=512)
    assert ws(**kw) == _records(8, 512, 32, 128, 64)
    # dk != dv: column-split carry
    kw = dict(B=1, HK=1, HV=2, dk=128, dv=64, chunk=16, T=32768)
    assert ws(**kw) == _records(1, 32768, 2, 128, 16)


def _gpu_visible():
    import torch

    return torch.cuda.device_count() > 0


@pytest.mark.skipif("_gpu_visible()", reason="valid fake pointers would reach a real GPU")
def test_valid_arguments_reach_the_runtime_without_a_gpu(L):
    # with no GPU, a call that passes validation fails at the first HIP call, cleanly
    assert prefill(L, dims(), ht=addr(5, 0)) == EHIP        # in-place ht == h0 is allowed
    assert decode(L, dims(T=1), ht=addr(5, 0)) == EHIP
    assert decode(L, dims(T=9, chunk=8), ht=addr(5, 0), entry="gdr_fused_recurrent") == EHIP
    assert tree(L, dims(T=64, dv=64)) == EHIP


def test_bench_carry_plan_matches_library(L):
    """bench.py reports which carry ran from a restatement of the library's shape rule;
    the workspace size (records, plus segment summaries and start states when segmented)
    shows the library's own choice, so the two must agree."""
    import bench

    mat = lambda dk: dk * dk * 4
    for B, HV, T, dk, C in [(1, 32, 4097, 128, 64), (1, 32, 32768, 128, 64), (8, 32, 512, 128, 64),
                            (2, 32, 4097, 128, 64), (4, 32, 4097, 64, 32), (2, 32, 512, 128, 64),
                            (2, 32, 4100, 64, 64), (3, 32, 3000, 128, 64), (1, 16, 20000, 128, 64),
                            (1, 2, 32768, 64, 16), (1, 2, 600, 64, 16), (1, 4, 9000, 32, 16)]:
        d = dims(B=B, HK=HV // 2 if HV > 1 else 1, HV=HV, dk=dk, dv=dk, chunk=C, T=T)
        got = L.gdr_chunk_prefill_workspace_bytes(ctypes.byref(d))
        plan = bench.carry_plan(B, T, HV, dk, dk, C)
        nseg = int(plan.split(", ")[1].split()[0]) if "segments" in plan else 1
        extra = B * HV * ((nseg - 1) * 2 * mat(dk) + nseg * mat(dk)) if nseg > 1 else 0
        assert got == _records(B, T, HV, dk, C) + extra, (B, HV, T, dk, C, plan)


def test_input_format_flags(L):
    """gdr_dims.flags: GDR_G_BF16 (bf16 q/k/v only), GDR_K_L2NORM, GDR_G_SOFTPLUS,
    GDR_G_PER_KEY_HEAD, GDR_O_BF16 and one of GDR_PREP_SPLIT (needs a per-key-head gate and
    HV/HK <= 8) or GDR_PREP_FUSED are defined; anything else is refused before any HIP call
    on every entry point."""
    for bad in (dict(flags=0x80), dict(flags=1 << 30), dict(flags=-1), dict(flags=1, qkv_dtype=1),
                dict(flags=7, qkv_dtype=1),
                dict(flags=0x10),                  # split prep without a per-key-head gate
                dict(flags=0x38),                  # split and fused both forced
                dict(flags=0x18, HK=1, HV=16)):    # split prep past its largest group (8)
        assert prefill(L, dims(**bad)) == EUNSUP, bad
        assert decode(L, dims(T=1, **bad)) == EUNSUP, bad
        assert decode(L, dims(T=3, **bad), entry="gdr_fused_recurrent") == EUNSUP, bad
        assert tree(L, dims(T=8, dv=64, **bad)) == EUNSUP, bad


def test_bf16_g_extent_in_alias_checks(L):
    """With GDR_G_BF16, g spans B*T*HV*dk*2 bytes: o over its last 16 bytes overlaps it."""
    gbytes = 2 * 5 * 4 * 64 * 2
    assert prefill(L, dims(flags=1), o=addr(3, gbytes - 16)) == EALIAS
    assert prefill(L, dims(flags=0), o=addr(3, 2 * gbytes - 16)) == EALIAS  # fp32 g: twice the bytes


def test_bf16_o_extent_in_alias_checks(L):
    """With GDR_O_BF16, o spans B*T*HV*dv*2 bytes: ht over its last 16 bytes overlaps it, ht
    right after it does not (which only an fp32 o would reach)."""
    obytes = 2 * 5 * 4 * 32 * 2
    assert prefill(L, dims(flags=0x40), ht=addr(6, obytes - 16)) == EALIAS
    assert prefill(L, dims(flags=0), ht=addr(6, obytes)) == EALIAS
    for entry in ("gdr_decode_step", "gdr_fused_recurrent"):
        assert decode(L, dims(T=1, flags=0x40), entry=entry, ht=addr(6, 2 * 4 * 32 * 2 - 16)) == EALIAS


@pytest.mark.skipif("_gpu_visible()", reason="valid fake pointers would reach a real GPU")
def test_bf16_o_valid_arguments_reach_the_runtime_without_a_gpu(L):
    obytes = 2 * 5 * 4 * 32 * 2
    assert prefill(L, dims(flags=0x40), ht=addr(6, obytes)) == EHIP
    assert prefill(L, dims(flags=0x41), ht=addr(6, obytes)) == EHIP  # with bf16 g
    assert decode(L, dims(T=1, flags=0x40, qkv_dtype=1), ht=addr(6, 2 * 4 * 32 * 2)) == EHIP
    assert tree(L, dims(T=8, dv=64, flags=0x40)) == EHIP


@pytest.mark.skipif("_gpu_visible()", reason="valid fake pointers would reach a real GPU")
def test_bf16_g_valid_arguments_reach_the_runtime_without_a_gpu(L):
    # o right after the bf16 g extent does not overlap it; the call passes validation and
    # fails only at the first HIP call
    gbytes = 2 * 5 * 4 * 64 * 2
    assert prefill(L, dims(flags=1), o=addr(3, gbytes)) == EHIP
    assert decode(L, dims(T=1, flags=1), ht=addr(5, 0)) == EHIP


def test_header_is_plain_c_and_links(L, tmp_path):
    """A C99 program using only include/gdr.h builds with gcc, links against libgdr.so and
    gets the documented host-side answers (no call in it reaches a GPU)."""
    src = os.path.join(ROOT, "tests", "c_abi", "abi_smoke.c")
    exe = str(tmp_path / "abi_smoke")
    libdir = os.path.dirname(gdr.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), src,
                    "-o", exe, "-L", libdir, "-lgdr", f"-Wl,-rpath,{libdir}"], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    assert "c abi ok" in res.stdout


@pytest.mark.skipif("_gpu_visible()", reason="valid fake pointers would reach a real GPU")
@pytest.mark.parametrize("flags", [2, 4, 6, 7, 3, 5])
def test_prologue_flags_pass_validation_without_a_gpu(L, flags):
    """The fused-prologue flags (alone, together, and with bf16 g) are accepted: with no GPU
    the call gets past every host check and fails only at the first HIP call."""
    assert prefill(L, dims(flags=flags)) == EHIP
    assert decode(L, dims(T=1, flags=flags)) == EHIP


@pytest.mark.skipif("_gpu_visible()", reason="valid fake pointers would reach a real GPU")
@pytest.mark.parametrize("flags", [0x8, 0x18, 0x28, 0x20, 0xF, 0x1F, 0x2F])
def test_gate_head_flags_pass_validation_without_a_gpu(L, flags):
    """A per-key-head gate and the prep-form flags are accepted on every entry point: with no
    GPU the call gets past every host check and fails only at the first HIP call."""
    assert prefill(L, dims(flags=flags)) == EHIP
    assert decode(L, dims(T=1, flags=flags)) == EHIP
    assert decode(L, dims(T=3, flags=flags), entry="gdr_fused_recurrent") == EHIP
    # the token-recurrence calls ignore the chunk length, zero included
    assert decode(L, dims(T=1, chunk=0, flags=flags)) == EHIP
    assert decode(L, dims(T=3, chunk=0, flags=flags), entry="gdr_fused_recurrent") == EHIP


def test_key_head_gate_extent_in_alias_checks(L):
    """With GDR_G_PER_KEY_HEAD, g spans B*T*HK*dk*4 bytes (half of the per-value-head extent
    at HV = 2 HK): o over its last 16 bytes overlaps it, o just past it does not."""
    gbytes = 2 * 5 * 2 * 64 * 4
    assert prefill(L, dims(flags=8), o=addr(3, gbytes - 16)) == EALIAS
    assert prefill(L, dims(flags=0), o=addr(3, gbytes + 16)) == EALIAS


def varlen_call(L, d, entry="gdr_chunk_prefill_varlen", ws_bytes=None, **ptrs):
    p = {n: addr(i) for i, n in enumerate(["cu", "q", "k", "v", "g", "beta", "h0", "o", "ht", "ws"])}
    p.update(ptrs)
    args = [p[n] for n in ("cu", "q", "k", "v", "g", "beta", "h0", "o", "ht")]
    if entry == "gdr_fused_recurrent_varlen":
        return L.gdr_fused_recurrent_varlen(ctypes.byref(d), *args, None)
    if ws_bytes is None:
        ws_bytes = L.gdr_chunk_prefill_varlen_workspace_bytes(ctypes.byref(d))
    return L.gdr_chunk_prefill_varlen(ctypes.byref(d), *args, p["ws"], ctypes.c_size_t(ws_bytes), None)


def test_varlen_workspace_bound(L):
    """Records for every chunk slot (T + N (C - 1)) / C per value head, then the plan
    (2 (N + 1) + slots int32)."""
    for N, T, C, dk in ((1, 1, 64, 128), (7, 4405, 64, 128), (4096, 4096, 16, 32), (3, 200, 32, 64)):
        d = dims(B=N, T=T, HK=2, HV=4, dk=dk, dv=dk, chunk=C)
        slots = (T + N * (C - 1)) // C
        rec = ((C // 16) * (dk // 32) * 2 + (dk // 16) * ((C + 31) // 32) + 2 * (C // 16) * ((C + 31) // 32) + 1) * 1024
        assert L.gdr_chunk_prefill_varlen_workspace_bytes(ctypes.byref(d)) == slots * 4 * rec + (2 * (N + 1) + slots) * 4
    assert L.gdr_chunk_prefill_varlen_workspace_bytes(ctypes.byref(dims(B=4097, T=5000))) == 0


def test_varlen_checks(L):
    for entry in ("gdr_chunk_prefill_varlen", "gdr_fused_recurrent_varlen"):
        assert varlen_call(L, dims(), entry, cu=None) == ENULL
        assert varlen_call(L, dims(), entry, cu=addr(0, 2)) == EALIGN
        assert varlen_call(L, dims(B=4097, T=5000), entry) == ESHAPE
        # o over the boundary array
        assert varlen_call(L, dims(), entry, o=addr(0, 0)) == EALIAS
    # the workspace must hold the plan too
    d = dims()
    need = L.gdr_chunk_prefill_varlen_workspace_bytes(ctypes.byref(d))
    assert varlen_call(L, d, ws_bytes=need - 4) == EWS


@pytest.mark.skipif("_gpu_visible()", reason="valid fake pointers would reach a real GPU")
def test_varlen_valid_arguments_reach_the_runtime_without_a_gpu(L):
    """States are [N][HV][dk][dv] and token tensors [T][..]: with N = 2, T = 5 every check
    passes and the call fails only at the first HIP call."""
    for entry in ("gdr_chunk_prefill_varlen", "gdr_fused_recurrent_varlen"):
        assert varlen_call(L, dims(), entry) == EHIP
        assert varlen_call(L, dims(flags=0x18), entry) == EHIP
