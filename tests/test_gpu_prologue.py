"""The fused input prologue on every entry point: raw keys (GDR_K_L2NORM) and gate logits
(GDR_G_SOFTPLUS) given to the kernels, against the fp64 oracle run on the keys normalised
and the logits mapped to -softplus in fp64 (oracle.l2_normalize_keys, oracle.neg_softplus)."""
import pytest
import torch

import gated_delta_rule_70_amd as gdr
import oracle
from gdr_synth import make_tree
from gpu_util import TOL, dev, err, note, small_inputs

pytestmark = pytest.mark.gpu


def raw_inputs(B, T, HK, HV, dk, dv, dtype=torch.bfloat16, seed=0, g_dtype=torch.float32):
    """The recipe's inputs with un-normalised keys (each row scaled by a factor in [0.1, 10])
    and gate logits a ~ N(0, 1) in place of g."""
    x = small_inputs(B, T, HK, HV, dk, dv, dtype=dtype, seed=seed)
    gen = torch.Generator("cpu").manual_seed(seed + 1000)
    scale = torch.exp(torch.empty(B, T, HK, 1).uniform_(-2.3, 2.3, generator=gen))
    x["k"] = (x["k"].float() * scale).to(dtype)
    x["g"] = torch.randn(B, T, HV, dk, generator=gen).to(g_dtype)
    return x


def reference(x, flags):
    kk, gg = x["k"], x["g"]
    if "k" in flags:
        kk = oracle.l2_normalize_keys(kk)
    if "g" in flags:
        gg = oracle.neg_softplus(gg)
    return oracle.sequential(x["q"], kk, x["v"], gg, x["beta"], x["h0"])


def kw(flags):
    return dict(k_l2norm="k" in flags, g_softplus="g" in flags)


FLAGS = ["kg", "k", "g"]


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("case", [(2, 150, 2, 4, 128, 128, 64), (1, 77, 2, 4, 64, 32, 16),
                                  (2, 70, 40, 80, 128, 128, 32)],
                         ids=["split_c64", "split_c16", "whole_head"])
def test_prefill_prologue(case, flags):
    B, T, HK, HV, dk, dv, C = case
    x = raw_inputs(B, T, HK, HV, dk, dv, seed=T + C)
    if "k" not in flags:
        x["k"] = small_inputs(B, T, HK, HV, dk, dv, seed=T + C)["k"]
    if "g" not in flags:
        x["g"] = small_inputs(B, T, HK, HV, dk, dv, seed=T + C)["g"]
    o_ref, ht_ref = reference(x, flags)
    d = dev(x)
    note(f"prologue prefill {case} flags={flags}")
    o, ht = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C, **kw(flags))
    torch.cuda.synchronize()
    eo, es = err(o, o_ref), err(ht, ht_ref)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


@pytest.mark.parametrize("dtype,g_dtype", [(torch.bfloat16, torch.float32), (torch.bfloat16, torch.bfloat16),
                                           (torch.float32, torch.float32)], ids=["bf16", "bf16_g_bf16", "fp32"])
def test_prologue_dtypes_all_entries(dtype, g_dtype):
    B, T, HK, HV, dk, dv = 2, 40, 2, 4, 128, 64
    x = raw_inputs(B, T, HK, HV, dk, dv, dtype=dtype, seed=31, g_dtype=g_dtype)
    o_ref, ht_ref = reference(x, "kg")
    d = dev(x)
    note(f"prologue all entries {dtype} g {g_dtype}")
    o1, h1 = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=32, **kw("kg"))
    o2, h2 = gdr.fused_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], **kw("kg"))
    o3, h3 = gdr.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=32, **kw("kg"))
    torch.cuda.synchronize()
    for name, (o, ht) in {"prefill": (o1, h1), "fused": (o2, h2), "forward": (o3, h3)}.items():
        eo, es = err(o, o_ref), err(ht, ht_ref)
        assert eo < TOL and es < TOL, f"{name}: o {eo:.2e} state {es:.2e}"


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("dk", [32, 64, 128])
def test_decode_prologue(flags, dk):
    x = raw_inputs(4, 1, 2, 4, dk, 128, seed=dk + len(flags))
    o_ref, ht_ref = reference(x, flags)
    d = dev(x)
    state = d["h0"].clone()
    note(f"prologue decode dk={dk} flags={flags}")
    o = gdr.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, **kw(flags))
    torch.cuda.synchronize()
    assert err(o, o_ref) < TOL and err(state, ht_ref) < TOL


@pytest.mark.parametrize("kind", ["chain", "random", "binary"])
def test_tree_verify_prologue(kind):
    B, T, HK, HV, dk, dv = 2, 64, 2, 4, 128, 64
    x = raw_inputs(B, T, HK, HV, dk, dv, seed=71)
    par = make_tree(B, T, kind, seed=3)
    ref = oracle.tree(x["q"], oracle.l2_normalize_keys(x["k"]), x["v"], oracle.neg_softplus(x["g"]), x["beta"],
                      x["h0"], parent=par.numpy())
    d = dev(x)
    note(f"prologue tree verify {kind}")
    o = gdr.tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], par.cuda(), h0=d["h0"], **kw("kg"))
    torch.cuda.synchronize()
    assert err(o, ref) < TOL


def test_noalloc_prologue():
    x = raw_inputs(1, 100, 2, 4, 128, 128, seed=91)
    o_ref, ht_ref = reference(x, "kg")
    d = dev(x)
    note("prologue noalloc prefill")
    o, ht = gdr.chunk_prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=64, **kw("kg"))
    torch.cuda.synchronize()
    assert err(o, o_ref) < TOL and err(ht, ht_ref) < TOL


def test_tree_verify_prologue_grouped_blocks():
    """Raw keys and gate logits on the tree path where a workgroup serves four column blocks
    of a head (B=8, HV=32, 128x128)."""
    B, T, HK, HV, dk, dv = 8, 64, 16, 32, 128, 128
    x = raw_inputs(B, T, HK, HV, dk, dv, seed=83)
    par = make_tree(B, T, "random", seed=5)
    ref = oracle.tree(x["q"], oracle.l2_normalize_keys(x["k"]), x["v"], oracle.neg_softplus(x["g"]), x["beta"],
                      x["h0"], parent=par.numpy())
    d = dev(x)
    note("prologue tree verify, grouped column blocks")
    o = gdr.tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], par.cuda(), h0=d["h0"], **kw("kg"))
    torch.cuda.synchronize()
    assert err(o, ref) < TOL
