"""Tree-verify solve (gdr_tree_verify) on the GPU against the fp64 oracle's tree route."""
import pytest
import torch

import gated_delta_rule_70_amd as gdr
import oracle
from gdr_synth import make_inputs, make_tree
from gpu_util import TOL, dev, err, note

pytestmark = pytest.mark.gpu


def _case(B, T, HK, HV, dk, dv, kind, seed, dtype=torch.bfloat16, h0=True):
    x = make_inputs(B, T, HK, HV, dk, dv, dtype=dtype, seed=seed, h0=h0)
    par = make_tree(B, T, kind, seed=seed)
    return x, par


@pytest.mark.parametrize("kind", ["chain", "star", "random", "binary"])
@pytest.mark.parametrize("T", [1, 5, 16, 33, 49, 64])
def test_tree_vs_oracle(kind, T):
    x, par = _case(2, T, 2, 4, 128, 128, kind, seed=200 + T)
    ref = oracle.tree(**x, parent=par.numpy())
    d = dev(x)
    note(f"tree {kind} T={T} 128x128")
    o = gdr.tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], par.cuda(), h0=d["h0"])
    torch.cuda.synchronize()
    assert err(o, ref) < TOL, f"{err(o, ref):.2e}"


@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 128), (64, 64), (128, 32), (64, 128)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_tree_dims_dtypes(dk, dv, dtype):
    G = 2 if dk == dv else 1
    x, par = _case(2, 37, 2, 2 * G, dk, dv, "random", seed=dk + dv, dtype=dtype, h0=(dk != 32))
    ref = oracle.tree(**x, parent=par.numpy())
    d = dev(x)
    note(f"tree random T=37 dk={dk} dv={dv} {dtype} G={G}")
    o = gdr.tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], par.cuda(), h0=d["h0"])
    torch.cuda.synchronize()
    assert err(o, ref) < TOL, f"{err(o, ref):.2e}"


def test_tree_chain_equals_prefill():
    x, par = _case(2, 50, 2, 4, 128, 128, "chain", seed=301)
    d = dev(x)
    note("tree chain vs chunked prefill and fused recurrence")
    o_t = gdr.tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], par.cuda(), h0=d["h0"])
    o_c, _ = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=64)
    o_r, _ = gdr.fused_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"])
    torch.cuda.synchronize()
    o_s, _ = oracle.sequential(**x)
    assert err(o_t, o_s) < TOL and err(o_c, o_s) < TOL and err(o_r, o_s) < TOL


def test_tree_out_of_range_parents_read_as_roots():
    x, par = _case(1, 20, 1, 2, 64, 64, "random", seed=303)
    bad = par.clone()
    bad[0, 3] = 7        # not an earlier node
    bad[0, 9] = -5       # below -1
    bad[0, 15] = 15      # itself
    fixed = bad.clone()
    for t in (3, 9, 15):
        fixed[0, t] = -1
    ref = oracle.tree(**x, parent=fixed.numpy())
    d = dev(x)
    note("tree with out-of-range parents")
    o = gdr.tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], bad.cuda(), h0=d["h0"])
    torch.cuda.synchronize()
    assert err(o, ref) < TOL


def test_tree_batched_and_deterministic():
    x, par = _case(8, 64, 16, 32, 128, 128, "binary", seed=305)
    d = dev(x)
    note("tree B=8 T=64 HV=32 binary, twice")
    p = par.cuda()
    o1 = gdr.tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], p, h0=d["h0"])
    o2 = gdr.tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], p, h0=d["h0"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    sub = {n: (x[n][:2] if x[n] is not None else None) for n in x}
    ref = oracle.tree(**sub, parent=par[:2].numpy())
    assert err(o1[:2], ref) < TOL


@pytest.mark.parametrize("B,dtype,h0", [(4, torch.bfloat16, True), (8, torch.float32, False)],
                         ids=["two_blocks_per_group", "four_blocks_per_group"])
def test_tree_column_block_groups(B, dtype, h0):
    """With enough heads (B * HV * dv/32 >= 512 at dk = 128) a workgroup takes 2 or 4
    32-column blocks of one head and forms the decayed rows, A, P and the diagonal inverses
    once for them: every batch element and head against the oracle."""
    x, par = _case(B, 64, 16, 32, 128, 128, "random", seed=311 + B, dtype=dtype, h0=h0)
    d = dev(x)
    note(f"tree column-block groups B={B} {dtype} h0={h0}")
    o = gdr.tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], par.cuda(), h0=d["h0"])
    torch.cuda.synchronize()
    ref = oracle.tree(**x, parent=par.numpy())
    assert err(o, ref) < TOL
