"""bf16 log-decays (GDR_G_BF16), the I/O-lean input format, on every path.

The kernels widen each bf16 value of g exactly to fp32, so a call with bf16 g must give
bitwise the result of the same call with an fp32 g holding the same values; and the result
must match the fp64 oracle run on those values within the usual bar."""
import pytest
import torch

import gated_delta_rule_70_amd as gdr
import oracle
from gdr_synth import PREFILL_1x4097, make_tree, workload_inputs
from gpu_util import TOL, dev, err, note, oracle_on_groups, sampled_groups, small_inputs

pytestmark = pytest.mark.gpu


def lean(x):
    """Inputs with g rounded to bf16 (bf16 copy for the GPU, the same values in fp32 for the
    fp32-g call and the oracle)."""
    x = dict(x)
    x["g"] = x["g"].to(torch.bfloat16).float()
    return x


def pair(d):
    """The device inputs twice: g as bf16 and as fp32 (same values)."""
    d16 = dict(d)
    d16["g"] = d["g"].to(torch.bfloat16)
    return d16, d


# (B, T, HK, HV, dk, chunk): column-split carry, whole-head carry (> 128 heads), segmented
PREFILL_CASES = [(2, 97, 2, 4, 128, 64), (2, 130, 2, 4, 64, 16), (2, 70, 40, 80, 128, 64),
                 (1, 8192, 1, 2, 64, 16)]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "B{}T{}HV{}dk{}C{}".format(c[0], c[1], c[3], c[4], c[5]))
def test_prefill_bf16_g_bitwise_and_parity(case):
    B, T, HK, HV, dk, C = case
    x = lean(small_inputs(B, T, HK, HV, dk, dk, seed=T + HV + C))
    d16, d32 = pair(dev(x))
    note(f"prefill bf16 g {case}")
    o16, h16 = gdr.chunk_prefill(d16["q"], d16["k"], d16["v"], d16["g"], d16["beta"], h0=d16["h0"], chunk=C)
    o32, h32 = gdr.chunk_prefill(d32["q"], d32["k"], d32["v"], d32["g"], d32["beta"], h0=d32["h0"], chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32) and torch.equal(h16, h32)
    o_ref, ht_ref = oracle.sequential(**x)
    assert err(o16, o_ref) < TOL and err(h16, ht_ref) < TOL


@pytest.mark.parametrize("T", [1, 5])
def test_token_paths_bf16_g_bitwise_and_parity(T):
    x = lean(small_inputs(3, T, 2, 4, 128, 128, seed=71 + T))
    d16, d32 = pair(dev(x))
    note(f"decode / fused recurrent bf16 g T={T}")
    o16, h16 = gdr.fused_recurrent(d16["q"], d16["k"], d16["v"], d16["g"], d16["beta"], h0=d16["h0"])
    o32, h32 = gdr.fused_recurrent(d32["q"], d32["k"], d32["v"], d32["g"], d32["beta"], h0=d32["h0"])
    torch.cuda.synchronize()
    assert torch.equal(o16, o32) and torch.equal(h16, h32)
    o_ref, ht_ref = oracle.sequential(**x)
    assert err(o16, o_ref) < TOL and err(h16, ht_ref) < TOL
    if T == 1:
        s = d16["h0"].clone()
        od = gdr.decode_step(d16["q"], d16["k"], d16["v"], d16["g"], d16["beta"], s)
        torch.cuda.synchronize()
        assert torch.equal(od, o16) and torch.equal(s, h16)


def test_tree_bf16_g_bitwise_and_parity():
    B, T = 2, 49
    x = lean(small_inputs(B, T, 2, 4, 128, 64, seed=73))
    par = make_tree(B, T, "random", seed=5)
    d16, d32 = pair(dev(x))
    p = par.cuda()
    note("tree verify bf16 g")
    o16 = gdr.tree_verify(d16["q"], d16["k"], d16["v"], d16["g"], d16["beta"], p, h0=d16["h0"])
    o32 = gdr.tree_verify(d32["q"], d32["k"], d32["v"], d32["g"], d32["beta"], p, h0=d32["h0"])
    torch.cuda.synchronize()
    assert torch.equal(o16, o32)
    o_ref = oracle.tree(**x, parent=par.numpy())
    assert err(o16, o_ref) < TOL


def test_headline_workload_bf16_g_sampled():
    """The single-sequence prefill (B=1, T=4097, HV=32, 128x128) with bf16 g, in the
    launch configuration the benchmark times; sampled key-head groups against the oracle."""
    w = PREFILL_1x4097
    x = lean(workload_inputs(w))
    d = dev(x)
    d["g"] = d["g"].to(torch.bfloat16)
    note("prefill_b1_t4097 with bf16 g")
    o, ht = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=None, chunk=w.chunk)
    torch.cuda.synchronize()
    G = w.HV // w.HK
    groups = sampled_groups(w.B, w.HK, 3, seed=w.seed)
    ref = oracle_on_groups(x, groups, G)
    oc, hc = o.cpu(), ht.cpu()
    for (b, kh), (o_r, ht_r) in ref.items():
        hv = slice(kh * G, (kh + 1) * G)
        assert err(oc[b, :, hv], o_r) < TOL and err(hc[b, hv], ht_r) < TOL, (b, kh)
