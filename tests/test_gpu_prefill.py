"""Chunked prefill on the GPU against the fp64 oracle: small shapes that span several
16-row blocks and chunks with ragged tails, the five measured workloads (sampled head
groups at full size), and the structural invariants of the method."""
import numpy as np
import pytest
import torch

import gated_delta_rule_70_amd as gdr
import oracle
from gdr_synth import (PREFILL_1x4097, PREFILL_1x32768, PREFILL_2x4097, PREFILL_8x97, PREFILL_8x512, TINY,
                       workload_inputs)
from gpu_util import (TOL, bf16_exact_unit_keys, dev, err, note, oracle_on_groups, sampled_groups, small_inputs,
                      token_err)

pytestmark = pytest.mark.gpu


def run_prefill(d, chunk, h0=True, **kw):
    return gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"],
                             h0=d["h0"] if h0 else None, chunk=chunk, **kw)


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 15, 17, 33, 64, 97, 130])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_small_128(C, T, dtype):
    x = small_inputs(2, T, 2, 4, 128, 128, dtype=dtype, seed=T + C)
    o_ref, ht_ref = oracle.sequential(**x)
    note(f"prefill dk=dv=128 C={C} T={T} {dtype}")
    o, ht = run_prefill(dev(x), C)
    torch.cuda.synchronize()
    eo, es = err(o, o_ref), err(ht, ht_ref)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 128), (64, 64), (64, 32), (128, 32), (128, 64)])
@pytest.mark.parametrize("C", [16, 64])
@pytest.mark.parametrize("G", [1, 2])
@pytest.mark.parametrize("h0", [True, False])
def test_prefill_head_dims(dk, dv, C, G, h0):
    x = small_inputs(2, 77, 2, 2 * G, dk, dv, seed=dk * 3 + dv + C + G, h0=h0)
    o_ref, ht_ref = oracle.sequential(**x)
    note(f"prefill dk={dk} dv={dv} C={C} G={G} h0={h0}")
    o, ht = run_prefill(dev(x), C, h0=h0)
    torch.cuda.synchronize()
    eo, es = err(o, o_ref), err(ht, ht_ref)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


def test_tiny_workload_full():
    """Tiny prefill, all fp32: B=1, HK=1, HV=2, T=64, dk=dv=32, chunk 16, h0 = 0."""
    w = TINY
    x = workload_inputs(w)
    o_ref, ht_ref = oracle.sequential(**x)
    note("tiny workload")
    o, ht = run_prefill(dev(x), w.chunk, h0=False)
    torch.cuda.synchronize()
    assert err(o, o_ref) < TOL and err(ht, ht_ref) < TOL


@pytest.mark.parametrize("w", [PREFILL_1x4097, PREFILL_8x512, PREFILL_8x97, PREFILL_1x32768, PREFILL_2x4097],
                         ids=lambda w: w.name)
def test_measured_workloads_all_heads(w):
    """Full-size runs in the benchmark's launch configuration, every (batch, value head)
    compared with the oracle on every output and on the final state; the per-token bar is
    logged beside the whole-tensor one."""
    x = workload_inputs(w)
    d = dev(x)
    note(f"workload {w.name}")
    o, ht = run_prefill(d, w.chunk, h0=w.h0)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(ht).all()
    o_ref, ht_ref = oracle.sequential(**x)
    eo, es = err(o, o_ref), err(ht, ht_ref)
    print(f"{w.name}: o {eo:.2e} state {es:.2e} per-token o {token_err(o, o_ref):.2e}")
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


def test_split_sequence_carry():
    x = small_inputs(2, 200, 2, 4, 128, 128, seed=21)
    d = dev(x)
    note("split sequence")
    o, ht = run_prefill(d, 64)
    first = {n: (t[:, :83].contiguous() if n != "h0" else t) for n, t in d.items()}
    o1, ht1 = run_prefill(first, 64)
    second = {n: (t[:, 83:].contiguous() if n != "h0" else ht1) for n, t in d.items()}
    o2, ht2 = run_prefill(second, 64)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.sequential(**x)
    assert err(torch.cat([o1, o2], 1), o_ref) < TOL and err(ht2, ht_ref) < TOL
    assert err(o, o_ref) < TOL and err(ht, ht_ref) < TOL


def test_prefill_then_decode_matches_concatenation():
    x = small_inputs(2, 70, 2, 4, 128, 128, seed=23)
    d = dev(x)
    note("prefill + decode")
    pre = {n: (t[:, :66].contiguous() if n != "h0" else t) for n, t in d.items()}
    o_p, state = run_prefill(pre, 64)
    outs = [o_p]
    for t in range(66, 70):
        outs.append(gdr.decode_step(*(d[n][:, t:t + 1].contiguous() for n in ("q", "k", "v", "g", "beta")),
                                    state))
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.sequential(**x)
    assert err(torch.cat(outs, 1), o_ref) < TOL and err(state, ht_ref) < TOL


def test_in_place_state_and_canaries():
    x = small_inputs(2, 97, 2, 4, 128, 128, seed=25)
    d = dev(x)
    o_ref, ht_ref = oracle.sequential(**x)
    need = gdr.workspace_bytes(2, 97, 2, 4, 128, 128, chunk=64)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda").fill_(0xFF)   # NaN-pattern halves
    o = torch.full((2, 97, 4, 128), float("nan"), device="cuda")
    state = d["h0"].clone()
    note("in-place state + canaries")
    gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=state, ht=state, o=o,
                      workspace=ws, chunk=64)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    assert err(o, o_ref) < TOL and err(state, ht_ref) < TOL


def test_prefill_deterministic():
    x = small_inputs(2, 150, 2, 4, 128, 128, seed=27)
    d = dev(x)
    note("prefill determinism")
    o1, h1 = run_prefill(d, 64)
    o2, h2 = run_prefill(d, 64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_prefill_exact_write_real_shape():
    # beta = 1, unit keys exact in bf16/fp16, q = k: every output equals its v exactly in
    # exact arithmetic, whatever the decay and initial state
    B, T, HK, HV = 1, 130, 2, 4
    x = small_inputs(B, T, HK, HV, 128, 128, seed=29)
    k = bf16_exact_unit_keys(B, T, HK, 128, seed=4).to(torch.bfloat16)
    x["k"], x["q"] = k, k.clone()
    x["beta"] = torch.ones_like(x["beta"])
    note("prefill exact write")
    o, _ = run_prefill(dev(x), 64)
    torch.cuda.synchronize()
    assert err(o, x["v"].double().numpy()) < TOL


def test_chunk_size_invariance():
    x = small_inputs(1, 160, 2, 4, 64, 64, seed=31)
    d = dev(x)
    note("chunk size invariance")
    res = [run_prefill(d, C) for C in (16, 32, 64)]
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.sequential(**x)
    for o, ht in res:
        assert err(o, o_ref) < TOL and err(ht, ht_ref) < TOL


# (B, T, HK, HV, dk, dv, chunk, dtype): column tiles per carry workgroup in the comment
MULTI_TILE = [(2, 300, 16, 32, 128, 128, 64, torch.bfloat16),   # 512 tiles: 2 per workgroup
              (3, 200, 16, 32, 128, 128, 32, torch.bfloat16),   # 768 tiles: 4
              (4, 150, 8, 32, 64, 64, 16, torch.float32),       # 512 tiles, chunk 16: 2
              (4, 130, 16, 32, 128, 64, 64, torch.bfloat16),    # dk != dv, 512 tiles: 2
              (2, 4097, 16, 32, 128, 128, 64, torch.bfloat16)]  # the B=2 T=4097 shape: 2


@pytest.mark.parametrize("case", MULTI_TILE, ids=lambda c: "B{}T{}HV{}_{}x{}C{}".format(*c[:2], *c[3:7]))
def test_column_split_multi_tile(case):
    """Between 32 and 128 (batch, head) pairs at dv = 128 (or more tiles than 256 at other
    shapes) the column-split carry takes 2 or 4 column tiles per workgroup so the grid stays
    within 256 workgroups; sampled key-head groups (the first and last among them) against
    the oracle, outputs and final state."""
    B, T, HK, HV, dk, dv, C, dt = case
    x = small_inputs(B, T, HK, HV, dk, dv, dtype=dt, seed=T + HV + C)
    need = gdr.workspace_bytes(B, T, HK, HV, dk, dv, C)
    assert need == B * HV * (-(-T // C)) * gdr.workspace_bytes(1, C, 1, 1, dk, dv, C)  # records only
    note(f"multi-tile column split {case}")
    d = dev(x)
    o, ht = run_prefill(d, C)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(ht).all()
    G = HV // HK
    groups = sampled_groups(B, HK, 3, seed=T)
    ref = oracle_on_groups(x, groups, G)
    for (b, kh), (o_r, ht_r) in ref.items():
        hv = slice(kh * G, (kh + 1) * G)
        eo, es = err(o[b, :, hv].cpu(), o_r), err(ht[b, hv].cpu(), ht_r)
        assert eo < TOL and es < TOL, f"group {(b, kh)}: o {eo:.2e} state {es:.2e}"


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("mode", ["h0", "no_h0", "in_place"])
def test_segmented_carry(dk, mode):
    """Two heads and 2048 chunks: the carry cuts the sequence into 128 segments of 16
    chunks, summarises each, combines the summaries in order and re-runs every segment
    from its start state; the result must still be the sequential recurrence.  The decay
    is slowed (g / 100) so each segment's transition matrix is far from zero and the
    combine step carries real weight."""
    T, C = 32768, 16
    x = small_inputs(1, T, 1, 2, dk, dk, seed=dk + len(mode), h0=mode != "no_h0")
    x["g"] = x["g"] / 100
    o_ref, ht_ref = oracle.sequential(**x)
    d = dev(x)
    note(f"segmented carry T={T} C={C} dk={dk} {mode}")
    if mode == "in_place":
        state = d["h0"].clone()
        o, _ = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=state, ht=state, chunk=C)
        ht = state
    else:
        o, ht = run_prefill(d, C, h0=mode == "h0")
    torch.cuda.synchronize()
    eo, es = err(o, o_ref), err(ht, ht_ref)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("T", [33, 97])
@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("h0", [True, False])
def test_wide_carry_many_heads(C, T, dk, h0):
    """More than 128 (batch, head) pairs: the carry runs one whole-head workgroup per head."""
    x = small_inputs(2, T, 40, 80, dk, dk, seed=C + T + dk + h0, h0=h0)
    o_ref, ht_ref = oracle.sequential(**x)
    note(f"wide carry B=2 HV=80 T={T} C={C} dk={dk} h0={h0}")
    o, ht = run_prefill(dev(x), C, h0=h0)
    torch.cuda.synchronize()
    eo, es = err(o, o_ref), err(ht, ht_ref)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


def test_wide_carry_fp32_inputs():
    x = small_inputs(2, 70, 40, 80, 128, 128, dtype=torch.float32, seed=3)
    o_ref, ht_ref = oracle.sequential(**x)
    note("wide carry fp32 q/k/v")
    o, ht = run_prefill(dev(x), 64)
    torch.cuda.synchronize()
    eo, es = err(o, o_ref), err(ht, ht_ref)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


@pytest.mark.parametrize("dk", [64, 128])
def test_segmented_carry_fp32_inputs(dk):
    """The segmented carry with fp32 q/k/v (the summary and full passes load v rows in
    fp32): 2 heads, 2048 chunks of 16, 128 segments, slowed decay."""
    x = small_inputs(1, 32768, 1, 2, dk, dk, dtype=torch.float32, seed=97 + dk)
    x["g"] = x["g"] / 100
    o_ref, ht_ref = oracle.sequential(**x)
    note(f"segmented carry fp32 q/k/v dk={dk}")
    o, ht = run_prefill(dev(x), 16)
    torch.cuda.synchronize()
    eo, es = err(o, o_ref), err(ht, ht_ref)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


def test_maximum_length_prefill():
    """The longest sequence one prefill launch takes at HV=32, 128x128, chunk 64 (T = 131007:
    one batch element's g and o rows, padding included, just under 2^31 bytes), so every
    31-bit buffer offset in the kernels is exercised near its limit; the carry runs in 8
    segments of 256 chunks.  One key-head group against the oracle."""
    B, T, HK, HV, dk = 1, 131007, 16, 32, 128
    assert (T + 64) * HV * dk * 4 < 2 ** 31 <= (T + 1 + 64) * HV * dk * 4  # T + 1 runs in windows
    x = small_inputs(B, T, HK, HV, dk, dk, seed=101)
    note(f"maximum-length prefill T={T}")
    d = dev(x)
    o, ht = run_prefill(d, 64)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(ht).all()
    G = HV // HK
    kh = HK - 1  # the last key head: the largest offsets
    ref = oracle_on_groups(x, [(0, kh)], G)
    o_r, ht_r = ref[(0, kh)]
    hv = slice(kh * G, (kh + 1) * G)
    eo, es = err(o[0, :, hv].cpu(), o_r), err(ht[0, hv].cpu(), ht_r)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


def test_windowed_prefill_equals_chained_calls():
    """Past what one launch addresses, the prefill runs as a chain of windows of W = 130944
    tokens (HV=32, 128x128, chunk 64), one batch element at a time.  Two elements of 131100
    tokens: bitwise the same outputs and final state as separate calls on each window with
    the state handed on by hand; the stateless and in-place forms give the same outputs; the
    last key-head group of the second element against the oracle."""
    B, T, HK, HV, dk, W = 2, 131100, 16, 32, 128, 130944
    assert (T + 64) * HV * dk * 4 >= 2 ** 31 > (W + 64) * HV * dk * 4
    x = small_inputs(B, T, HK, HV, dk, dk, seed=103)
    note(f"windowed prefill B={B} T={T}")
    d = dev(x)
    o, ht = run_prefill(d, 64)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(ht).all()
    for b in range(B):
        h = d["h0"][b:b + 1]
        for t0, t1 in ((0, W), (W, T)):
            part = {n: d[n][b:b + 1, t0:t1].contiguous() for n in ("q", "k", "v", "g", "beta")}
            oc, h = gdr.chunk_prefill(part["q"], part["k"], part["v"], part["g"], part["beta"], h0=h, chunk=64)
            assert torch.equal(o[b:b + 1, t0:t1], oc), (b, t0)
            del part, oc
        assert torch.equal(ht[b:b + 1], h), b
    o_ref = o.clone()
    o2, none = run_prefill(d, 64, o=o, want_state=False)
    assert none is None and torch.equal(o2, o_ref)
    st = d["h0"].clone()
    run_prefill(d, 64, o=o, h0=False, want_state=False)  # o holds another result first
    gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=st, ht=st, o=o, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(st, ht)
    G = HV // HK
    kh = HK - 1
    ref = oracle_on_groups(x, [(1, kh)], G)
    o_r, ht_r = ref[(1, kh)]
    hv = slice(kh * G, (kh + 1) * G)
    eo, es = err(o[1, :, hv].cpu(), o_r), err(ht[1, hv].cpu(), ht_r)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


@pytest.mark.parametrize("case", [(2, 97, 2, 4, 128, 64), (2, 70, 40, 80, 128, 64), (1, 32768, 1, 2, 64, 16)],
                         ids=["column_split", "whole_head", "segmented"])
def test_two_stage_calls_equal_one_call(case):
    """gdr_chunk_prep followed by gdr_chunk_carry on the same workspace gives bitwise the
    result of gdr_chunk_prefill, on every carry path."""
    B, T, HK, HV, dk, C = case
    x = small_inputs(B, T, HK, HV, dk, dk, seed=T + HV)
    d = dev(x)
    note(f"two-stage prefill {case}")
    o1, h1 = run_prefill(d, C)
    ws = torch.empty(gdr.workspace_bytes(B, T, HK, HV, dk, dk, C), dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o1)
    h2 = torch.empty_like(h1)
    for stage in ("prep", "carry"):
        gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C, o=o2, ht=h2,
                          workspace=ws, stage=stage)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
