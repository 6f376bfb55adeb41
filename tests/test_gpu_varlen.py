"""Packed variable-length batches (gdr_chunk_prefill_varlen, gdr_fused_recurrent_varlen)
against the fp64 oracle run per sequence (oracle.varlen): sequences of 1, 15, 97 and 4097
rows (and empty ones, and exact multiples of the chunk) in one call, on both carry forms
(whole head with many (sequence, head) pairs, column split with few), both prep forms, and
the token recurrence.  Equal-length sequences packed must give bitwise the dense batch."""
import numpy as np
import pytest
import torch

import gated_delta_rule_70_amd as gdr
import oracle
from gdr_synth import make_inputs
from gpu_util import TOL, err, note

pytestmark = pytest.mark.gpu


def packed_inputs(lengths, HK, HV, dk, dv, dtype=torch.bfloat16, seed=0, h0=True, gate_heads="value"):
    T = sum(lengths)
    x = make_inputs(1, T, HK, HV, dk, dv, dtype=dtype, seed=seed, h0=False, gate_heads=gate_heads)
    x = {n: t[0].contiguous() for n, t in x.items() if t is not None}
    gen = torch.Generator("cpu").manual_seed(seed + 7)
    x["h0"] = (0.3 * torch.randn(len(lengths), HV, dk, dv, generator=gen)) if h0 else None
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    return x, cu


def gpu(x):
    return {n: (None if t is None else t.cuda()) for n, t in x.items()}


def check(o, ht, x, cu, lengths):
    o_ref, ht_ref = oracle.varlen(oracle.sequential, cu_seqlens=cu.numpy(), **x)
    o = o.detach().double().cpu().numpy()
    # every sequence on its own scale (a short sequence's outputs are not hidden by a long one's)
    for i in range(len(lengths)):
        a, b = int(cu[i]), int(cu[i + 1])
        if b > a:
            e = oracle.rel_err(o[a:b], o_ref[a:b])
            assert e < TOL, f"sequence {i} ({b - a} rows): o {e:.2e}"
        e = oracle.rel_err(ht[i].double().cpu().numpy(), ht_ref[i])
        assert e < TOL, f"sequence {i} ({b - a} rows): state {e:.2e}"


MIXED = [1, 15, 97, 4097, 0, 64, 130]


@pytest.mark.parametrize("prep", ["auto", "fused", "split"])
def test_prefill_varlen_mixed_lengths_whole_head(prep):
    """7 sequences x 32 value heads = 224 (sequence, head) pairs: the whole-head carry."""
    HK, HV, dk, dv, C = 16, 32, 128, 128, 64
    gh = "key" if prep == "split" else "value"
    x, cu = packed_inputs(MIXED, HK, HV, dk, dv, seed=11, gate_heads=gh)
    d = gpu(x)
    note(f"varlen prefill {MIXED} prep={prep}")
    o, ht = gdr.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu.cuda(), h0=d["h0"], chunk=C,
                                     prep=prep)
    torch.cuda.synchronize()
    check(o, ht, x, cu, MIXED)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("dims", [(128, 64), (64, 64), (32, 128)])
def test_prefill_varlen_column_split(dims, C, dtype):
    """Few (sequence, head) pairs: the column-split carry; ragged lengths around the chunk."""
    dk, dv = dims
    lengths = [1, C - 1, 0, 2 * C + 1, 97, C]
    x, cu = packed_inputs(lengths, 1, 2, dk, dv, dtype=dtype, seed=C + dk)
    d = gpu(x)
    note(f"varlen prefill column split {lengths} dk={dk} dv={dv} C={C} {dtype}")
    o, ht = gdr.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu.cuda(), h0=d["h0"], chunk=C)
    torch.cuda.synchronize()
    check(o, ht, x, cu, lengths)


@pytest.mark.parametrize("lengths,HV", [([1, 97, 300], 32), ([200, 0, 65, 1], 16)],
                         ids=["3x32_heads_4_tiles", "4x16_heads_2_tiles"])
def test_prefill_varlen_column_split_multi_tile(lengths, HV):
    """Between 32 and 128 (sequence, head) pairs at dv = 128: the column-split carry with
    4 (96 pairs) or 2 (64 pairs) column tiles per workgroup, sequences read from the plan."""
    x, cu = packed_inputs(lengths, HV // 2, HV, 128, 128, seed=sum(lengths) + HV)
    d = gpu(x)
    note(f"varlen prefill multi-tile column split {lengths} HV={HV}")
    o, ht = gdr.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu.cuda(), h0=d["h0"], chunk=64)
    torch.cuda.synchronize()
    check(o, ht, x, cu, lengths)


def test_prefill_varlen_zero_h0_and_no_state():
    lengths = [33, 1, 70]
    x, cu = packed_inputs(lengths, 2, 4, 128, 128, seed=5, h0=False)
    d = gpu(x)
    note("varlen prefill without h0, without ht")
    o, ht = gdr.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu.cuda(), chunk=64,
                                     want_state=False)
    torch.cuda.synchronize()
    assert ht is None
    o_ref, _ = oracle.varlen(oracle.sequential, cu_seqlens=cu.numpy(), **x)
    assert err(o, o_ref) < TOL


@pytest.mark.parametrize("fn", ["chunk_prefill", "fused_recurrent"])
def test_varlen_equal_lengths_bitwise_dense(fn):
    """8 sequences of 97 rows packed == the dense B=8 T=97 batch, bit for bit."""
    B, T, HK, HV, dk, dv = 8, 97, 16, 32, 128, 128
    x = make_inputs(B, T, HK, HV, dk, dv, seed=41, h0=True)
    d = gpu(x)
    cu = torch.arange(0, B * T + 1, T, dtype=torch.int32).cuda()
    flat = {n: (None if t is None else (t if n == "h0" else t.reshape(B * T, *t.shape[2:]))) for n, t in d.items()}
    note(f"varlen == dense bitwise ({fn})")
    if fn == "chunk_prefill":
        o1, h1 = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=64)
        o2, h2 = gdr.chunk_prefill_varlen(flat["q"], flat["k"], flat["v"], flat["g"], flat["beta"], cu,
                                          h0=flat["h0"], chunk=64)
    else:
        o1, h1 = gdr.fused_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"])
        o2, h2 = gdr.fused_recurrent_varlen(flat["q"], flat["k"], flat["v"], flat["g"], flat["beta"], cu,
                                            h0=flat["h0"])
    torch.cuda.synchronize()
    assert torch.equal(o1.reshape(B * T, HV, dv), o2) and torch.equal(h1, h2)


@pytest.mark.parametrize("lengths", [[1, 3, 8, 0, 5, 16], [2] * 40, [1]])
def test_fused_recurrent_varlen(lengths):
    x, cu = packed_inputs(lengths, 16, 32, 128, 128, seed=len(lengths))
    d = gpu(x)
    note(f"varlen fused recurrence {lengths[:8]}")
    o, ht = gdr.fused_recurrent_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu.cuda(), h0=d["h0"])
    torch.cuda.synchronize()
    check(o, ht, x, cu, lengths)


def test_varlen_prologue_flags():
    """Raw keys and gate logits per key head on a packed batch (split prep)."""
    lengths = [5, 200, 64, 1]
    HK, HV, dk, dv = 4, 8, 128, 128
    x, cu = packed_inputs(lengths, HK, HV, dk, dv, seed=21, gate_heads="key")
    gen = torch.Generator("cpu").manual_seed(22)
    T = sum(lengths)
    x["k"] = (x["k"].float() * torch.exp(torch.empty(T, HK, 1).uniform_(-2.3, 2.3, generator=gen))).to(x["k"].dtype)
    x["g"] = torch.randn(T, HK, dk, generator=gen)
    ref_in = dict(x, k=oracle.l2_normalize_keys(x["k"]), g=oracle.neg_softplus(x["g"]))
    d = gpu(x)
    note("varlen prefill with prologue, split prep")
    o, ht = gdr.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu.cuda(), h0=d["h0"], chunk=64,
                                     k_l2norm=True, g_softplus=True, prep="split")
    torch.cuda.synchronize()
    check(o, ht, ref_in, cu, lengths)
