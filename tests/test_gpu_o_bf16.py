"""bf16 outputs (GDR_O_BF16): every entry point computes each output in fp32 exactly as it
does for an fp32 o and rounds it to the nearest bf16 (ties to even) as it stores it.  So on
every path -- decode step, fused recurrence, routed call, tree verify, the chunked prefill
on each carry form (column split with one, two or four tiles per workgroup, whole head,
time segments), packed batches, and a sequence long enough to run in windows -- the bf16 o
must be bitwise the bf16 rounding of the same call's fp32 o, and the final states bitwise
the fp32 call's.  Against the fp64 oracle the bar widens by the rounding alone: each value
moves by at most 2^-8 of itself, so the relative error of the tensor is at most
TOL + 2^-8 (1 + TOL)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_70_amd as gdr
import oracle
from gdr_synth import make_inputs, make_tree
from gpu_util import TOL, dev, err, note, small_inputs

pytestmark = pytest.mark.gpu

TOL_BF16_O = TOL + 2.0 ** -8 * (1 + TOL)


def rne(o32):
    """fp32 outputs rounded to bf16, nearest even (torch's conversion on the host)."""
    return o32.detach().cpu().to(torch.bfloat16)


def same(o16, o32):
    assert o16.dtype == torch.bfloat16
    a = o16.detach().cpu().view(torch.int16)
    b = rne(o32).view(torch.int16)
    n = int((a != b).sum())
    assert n == 0, f"{n} of {a.numel()} outputs differ from the rounded fp32 outputs"


# (B, T, HK, HV, dk, dv, chunk, dtype): carry form in the comment
PREFILL = [(2, 97, 2, 4, 128, 128, 64, torch.bfloat16),     # column split, two wave roles
           (2, 300, 16, 32, 128, 128, 64, torch.bfloat16),  # column split, 2 tiles per workgroup
           (3, 200, 16, 32, 128, 128, 32, torch.bfloat16),  # column split, 4 tiles per workgroup
           (2, 77, 2, 4, 128, 64, 16, torch.bfloat16),      # dk != dv
           (2, 70, 40, 80, 128, 128, 64, torch.bfloat16),   # whole head (160 heads)
           (1, 32768, 1, 2, 64, 64, 16, torch.bfloat16),    # time segments (128)
           (2, 97, 2, 4, 64, 64, 32, torch.float32)]        # fp32 q/k/v


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "B{}T{}HV{}_{}x{}C{}_{}".format(
    c[0], c[1], c[3], c[4], c[5], c[6], str(c[7]).split(".")[-1]))
def test_prefill_bf16_o_is_rounded_fp32_o(case):
    B, T, HK, HV, dk, dv, C, dt = case
    x = small_inputs(B, T, HK, HV, dk, dv, dtype=dt, seed=T + HV + C)
    d = dev(x)
    note(f"bf16 o prefill {case}")
    o32, h32 = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C)
    o16, h16 = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C,
                                 out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    same(o16, o32)
    assert torch.equal(h16, h32)


def test_prefill_bf16_o_against_oracle():
    """bf16 o against the fp64 oracle within the widened bar; the final state (fp32) within
    the plain one."""
    x = small_inputs(2, 200, 2, 4, 128, 128, seed=71)
    o_ref, ht_ref = oracle.sequential(**x)
    d = dev(x)
    note("bf16 o prefill vs oracle")
    o16, ht = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=64,
                                out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    eo, es = err(o16.float(), o_ref), err(ht, ht_ref)
    assert eo < TOL_BF16_O and es < TOL, f"o {eo:.2e} state {es:.2e}"


def test_prefill_bf16_o_caller_buffer_and_stages():
    """A bf16 ``o`` passed in selects the format; the two stage calls and the
    allocation-free entry point give the same bits."""
    x = small_inputs(2, 130, 2, 4, 128, 128, seed=72)
    d = dev(x)
    note("bf16 o caller buffer, stages, noalloc")
    o1, h1 = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=64,
                               out_dtype=torch.bfloat16)
    o2 = torch.empty(o1.shape, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdr.workspace_bytes(2, 130, 2, 4, 128, 128, 64), dtype=torch.uint8, device="cuda")
    h2 = torch.empty_like(h1)
    for stage in ("prep", "carry"):
        gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=64, o=o2, ht=h2,
                          workspace=ws, stage=stage)
    o3, h3 = gdr.chunk_prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=64,
                                       out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2) and torch.equal(o1, o3) and torch.equal(h1, h3)


def test_token_paths_bf16_o():
    """Decode step, fused recurrence and the routed call on both of its paths."""
    x = small_inputs(3, 1, 2, 4, 128, 128, seed=73)
    d = dev(x)
    note("bf16 o decode")
    s32, s16 = d["h0"].clone(), d["h0"].clone()
    o32 = gdr.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], s32)
    o16 = gdr.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], s16, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    same(o16, o32)
    assert torch.equal(s16, s32)
    for T in (5, 100):
        x = small_inputs(2, T, 2, 4, 64, 128, seed=74 + T)
        d = dev(x)
        note(f"bf16 o fused recurrence / forward T={T}")
        if T <= gdr.RECURRENT_MAX_T:
            o32, h32 = gdr.fused_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"])
            o16, h16 = gdr.fused_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"],
                                           out_dtype=torch.bfloat16)
            same(o16, o32)
            assert torch.equal(h16, h32)
        o32, h32 = gdr.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=32)
        o16, h16 = gdr.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=32,
                               out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        same(o16, o32)
        assert torch.equal(h16, h32)


@pytest.mark.parametrize("kind", ["binary", "chain"])
def test_tree_verify_bf16_o(kind):
    x = make_inputs(2, 33, 2, 4, 128, 128, seed=75, h0=True)
    par = make_tree(2, 33, kind, seed=75).cuda()
    d = dev(x)
    note(f"bf16 o tree {kind}")
    o32 = gdr.tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], par, h0=d["h0"])
    o16 = gdr.tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], par, h0=d["h0"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    same(o16, o32)


@pytest.mark.parametrize("HV", [4, 32])
def test_packed_batch_bf16_o(HV):
    """Packed sequences (1, 15, 97, 300 rows, an empty one, 64): the chunked prefill (column
    split at 4 heads, whole head at 32) and the token recurrence."""
    lengths = [1, 15, 97, 300, 0, 64]
    T = sum(lengths)
    x = make_inputs(1, T, HV // 2, HV, 128, 128, seed=76 + HV, h0=False)
    x = {n: t[0].contiguous().cuda() for n, t in x.items() if t is not None}
    h0 = (0.3 * torch.randn(len(lengths), HV, 128, 128, generator=torch.Generator().manual_seed(3))).cuda()
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device="cuda")
    note(f"bf16 o packed HV={HV}")
    o32, h32 = gdr.chunk_prefill_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, h0=h0)
    o16, h16 = gdr.chunk_prefill_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, h0=h0,
                                        out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    same(o16, o32)
    assert torch.equal(h16, h32)
    o32, h32 = gdr.fused_recurrent_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, h0=h0)
    o16, h16 = gdr.fused_recurrent_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, h0=h0,
                                          out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    same(o16, o32)
    assert torch.equal(h16, h32)


def test_windowed_prefill_bf16_o():
    """A sequence past one launch (T = 131100 at HV = 32, 128x128: two windows), whose
    window offsets into o are in bf16 elements."""
    B, T, HK, HV, dk = 1, 131100, 16, 32, 128
    x = small_inputs(B, T, HK, HV, dk, dk, seed=77)
    d = dev(x)
    note(f"bf16 o windowed prefill T={T}")
    o32, h32 = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=64)
    o16, h16 = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=64,
                                 out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(h16, h32)
    # compared on the device in slices (the whole tensor is 537 M values)
    for t0 in range(0, T, 16384):
        a = o16[:, t0:t0 + 16384].view(torch.int16)
        b = o32[:, t0:t0 + 16384].to(torch.bfloat16).view(torch.int16)
        assert torch.equal(a, b), t0


@pytest.mark.parametrize("gate_heads", ["value", "key"])
def test_bf16_o_with_prologue_and_gate_heads(gate_heads):
    """bf16 o combined with raw keys and gate logits (the fused prologue) and with a gate per
    key head or per value head: the prefill (both prep forms where the gate is per key head)
    and the decode step, each bitwise the rounded fp32 o of the same call."""
    B, T, HK, HV, dk = 2, 150, 2, 8, 128
    x = make_inputs(B, T, HK, HV, dk, dk, seed=78, h0=True, gate_heads=gate_heads)
    gen = torch.Generator("cpu").manual_seed(79)
    scale = torch.exp(torch.empty(B, T, HK, 1).uniform_(-2.3, 2.3, generator=gen))
    x["k"] = (x["k"].float() * scale).to(torch.bfloat16)
    x["g"] = torch.randn(x["g"].shape, generator=gen)
    d = dev(x)
    flags = dict(k_l2norm=True, g_softplus=True)
    preps = ["fused", "split"] if gate_heads == "key" else ["auto"]
    for prep in preps:
        note(f"bf16 o with prologue, gate per {gate_heads} head, prep {prep}")
        o32, h32 = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=64, prep=prep,
                                     **flags)
        o16, h16 = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=64, prep=prep,
                                     out_dtype=torch.bfloat16, **flags)
        torch.cuda.synchronize()
        same(o16, o32)
        assert torch.equal(h16, h32)
    t1 = {n: (None if t is None else (t[:, :1].contiguous() if t.dim() >= 3 and n != "h0" else t))
          for n, t in d.items()}
    s32, s16 = d["h0"].clone(), d["h0"].clone()
    o32 = gdr.decode_step(t1["q"], t1["k"], t1["v"], t1["g"], t1["beta"], s32, **flags)
    o16 = gdr.decode_step(t1["q"], t1["k"], t1["v"], t1["g"], t1["beta"], s16, out_dtype=torch.bfloat16, **flags)
    torch.cuda.synchronize()
    same(o16, o32)
    assert torch.equal(s16, s32)
