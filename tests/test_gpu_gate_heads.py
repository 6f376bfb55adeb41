"""A gate shared per key head (g [B,T,HK,dk], beta per value head) on every entry point,
against the fp64 oracle with the gate expanded to its value heads (oracle.gate_per_value_head).
The prefill runs its chunk-parallel stage in both forms of the uzu PR #576 review thread on
the per-value-head gram: fused (one workgroup per value head) and split (one per key head,
the gram once per group, the solve per value head); the two must also agree bit for bit,
records included."""
import pytest
import torch

import gated_delta_rule_70_amd as gdr
import oracle
from gdr_synth import make_tree
from gpu_util import TOL, dev, err, note, small_inputs, token_err

pytestmark = pytest.mark.gpu


def key_gate_inputs(B, T, HK, HV, dk, dv, dtype=torch.bfloat16, seed=0, h0=True, g_dtype=torch.float32):
    x = small_inputs(B, T, HK, HV, dk, dv, dtype=dtype, seed=seed, h0=h0, gate_heads="key")
    x["g"] = x["g"].to(g_dtype)
    return x


CASES = [  # B, T, HK, HV, dk, dv, C
    (2, 150, 2, 4, 128, 128, 64),
    (1, 97, 1, 4, 128, 64, 32),
    (2, 77, 2, 16, 64, 64, 16),     # G = 8, the split form's largest group
    (1, 130, 3, 6, 32, 128, 64),
    (3, 40, 4, 4, 128, 128, 16),    # G = 1: the two layouts coincide
]


@pytest.mark.parametrize("prep", ["fused", "split", "auto"])
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}T{c[1]}HK{c[2]}HV{c[3]}dk{c[4]}dv{c[5]}C{c[6]}" for c in CASES])
def test_prefill_key_head_gate(case, prep):
    B, T, HK, HV, dk, dv, C = case
    x = key_gate_inputs(B, T, HK, HV, dk, dv, seed=T + HV)
    o_ref, ht_ref = oracle.sequential(**x)
    d = dev(x)
    note(f"key-head gate prefill {case} prep={prep}")
    o, ht = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C, prep=prep)
    torch.cuda.synchronize()
    eo, es = err(o, o_ref), err(ht, ht_ref)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


@pytest.mark.parametrize("dtype,g_dtype", [(torch.bfloat16, torch.float32), (torch.bfloat16, torch.bfloat16),
                                           (torch.float32, torch.float32)], ids=["bf16", "bf16_g16", "fp32"])
@pytest.mark.parametrize("C", [16, 32, 64])
def test_split_and_fused_agree_bitwise(C, dtype, g_dtype):
    """Same records and same outputs from both forms (the beta row scaling is the same fp32
    multiplication in both)."""
    B, T, HK, HV, dk, dv = 2, 3 * C + 5, 2, 4, 128, 128
    x = key_gate_inputs(B, T, HK, HV, dk, dv, dtype=dtype, g_dtype=g_dtype, seed=C)
    d = dev(x)
    nbytes = gdr.workspace_bytes(B, T, HK, HV, dk, dv, C, dtype)
    outs = {}
    for prep in ("fused", "split"):
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        note(f"bitwise split/fused C={C} {dtype} g {g_dtype} prep={prep}")
        o, ht = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C,
                                  workspace=ws, prep=prep)
        torch.cuda.synchronize()
        outs[prep] = (o, ht, ws)
    (o1, h1, w1), (o2, h2, w2) = outs["fused"], outs["split"]
    assert torch.equal(w1, w2), "records differ"
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


@pytest.mark.parametrize("flags", ["k", "g", "kg"])
def test_split_with_prologue(flags):
    """Raw keys and gate logits per key head, split form, against the oracle on the
    pre-processed inputs."""
    B, T, HK, HV, dk, dv, C = 2, 150, 2, 4, 128, 128, 64
    x = key_gate_inputs(B, T, HK, HV, dk, dv, seed=31)
    gen = torch.Generator("cpu").manual_seed(32)
    if "k" in flags:
        x["k"] = (x["k"].float() * torch.exp(torch.empty(B, T, HK, 1).uniform_(-2.3, 2.3, generator=gen))).to(x["k"].dtype)
    if "g" in flags:
        x["g"] = torch.randn(B, T, HK, dk, generator=gen)
    ref_in = dict(x)
    if "k" in flags:
        ref_in["k"] = oracle.l2_normalize_keys(x["k"])
    if "g" in flags:
        ref_in["g"] = oracle.neg_softplus(x["g"])
    o_ref, ht_ref = oracle.sequential(**ref_in)
    d = dev(x)
    note(f"split prep with prologue {flags}")
    o, ht = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C, prep="split",
                              k_l2norm="k" in flags, g_softplus="g" in flags)
    torch.cuda.synchronize()
    eo, es = err(o, o_ref), err(ht, ht_ref)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


@pytest.mark.parametrize("T", [1, 5, 16])
def test_token_paths_key_head_gate(T):
    """Decode step (T = 1) and the fused recurrence with a per-key-head gate."""
    B, HK, HV, dk, dv = 3, 2, 8, 128, 128
    x = key_gate_inputs(B, T, HK, HV, dk, dv, seed=50 + T)
    o_ref, ht_ref = oracle.sequential(**x)
    d = dev(x)
    note(f"key-head gate token paths T={T}")
    if T == 1:
        st = d["h0"].clone()
        o = gdr.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st)
        ht = st
    else:
        o, ht = gdr.fused_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"])
    torch.cuda.synchronize()
    eo, es = err(o, o_ref), err(ht, ht_ref)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


@pytest.mark.parametrize("kind", ["chain", "binary", "random"])
def test_tree_key_head_gate(kind):
    B, T, HK, HV, dk, dv = 2, 48, 2, 4, 128, 128
    x = key_gate_inputs(B, T, HK, HV, dk, dv, seed=61)
    par = make_tree(B, T, kind, seed=62)
    o_ref = oracle.tree(**x, parent=par.numpy())
    d = dev(x)
    note(f"key-head gate tree {kind}")
    o = gdr.tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], par.cuda(), h0=d["h0"])
    torch.cuda.synchronize()
    e = err(o, o_ref)
    assert e < TOL, f"o {e:.2e}"


@pytest.mark.parametrize("prep", ["fused", "split"])
def test_single_sequence_prefill_key_head_gate_all_heads(prep):
    """B=1 T=4097 HK=16 HV=32 dk=dv=128 C=64 with one gate per key head, every head against
    the oracle, plus the per-token bar on o."""
    B, T, HK, HV, dk, dv, C = 1, 4097, 16, 32, 128, 128, 64
    x = key_gate_inputs(B, T, HK, HV, dk, dv, seed=3, h0=False)
    o_ref, ht_ref = oracle.sequential(**x)
    d = dev(x)
    note(f"key-head gate single-sequence prefill prep={prep}")
    o, ht = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=C, prep=prep)
    torch.cuda.synchronize()
    eo, es, et = err(o, o_ref), err(ht, ht_ref), token_err(o, o_ref)
    print(f"prep={prep}: o {eo:.2e} state {es:.2e} per-token {et:.2e}")
    assert eo < TOL and es < TOL and et < 10 * TOL, f"o {eo:.2e} state {es:.2e} per-token {et:.2e}"


def test_split_rejected_where_it_does_not_apply():
    B, T, HK, HV, dk, dv = 1, 64, 1, 16, 64, 64  # G = 16 > 8
    x = dev(key_gate_inputs(B, T, HK, HV, dk, dv, seed=1, h0=False))
    with pytest.raises(gdr.GdrError):
        gdr.chunk_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], chunk=64, prep="split")
    o, _ = gdr.chunk_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], chunk=64, prep="auto")
    torch.cuda.synchronize()
    o_ref, _ = oracle.sequential(**{k: v.cpu() if v is not None else None for k, v in x.items()})
    assert err(o, o_ref) < TOL
    # a gate per value head cannot take the split form
    y = dev(small_inputs(1, 64, 2, 4, 64, 64, seed=2))
    with pytest.raises(gdr.GdrError):
        gdr.chunk_prefill(y["q"], y["k"], y["v"], y["g"], y["beta"], chunk=64, prep="split")
