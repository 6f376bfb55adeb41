"""Fused token recurrence (gdr_fused_recurrent: T tokens in one launch, the state held on
chip) on the GPU, against the fp64 oracle and against the library's other two paths."""
import pytest
import torch

import gated_delta_rule_70_amd as gdr
import oracle
from gdr_synth import DECODE, make_inputs
from gpu_util import TOL, dev, err, note, oracle_on_groups, sampled_groups, small_inputs

pytestmark = pytest.mark.gpu

DIMS = [(32, 32), (32, 128), (64, 64), (128, 32), (128, 128)]


@pytest.mark.parametrize("T", [1, 2, 7, 16, 33])
@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_recurrent_vs_oracle(T, dk, dv, dtype):
    G = 2 if (dk + dv) % 64 == 0 else 1
    x = small_inputs(2, T, 2, 2 * G, dk, dv, dtype=dtype, seed=100 + T + dk + dv, h0=(T % 2 == 1))
    o_ref, ht_ref = oracle.sequential(**x)
    d = dev(x)
    note(f"recurrent T={T} dk={dk} dv={dv} {dtype} G={G} h0={x['h0'] is not None}")
    o, ht = gdr.fused_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"])
    torch.cuda.synchronize()
    assert err(o, o_ref) < TOL, f"o {err(o, o_ref):.2e}"
    assert err(ht, ht_ref) < TOL, f"state {err(ht, ht_ref):.2e}"


def test_recurrent_equals_successive_decode_steps_bitwise():
    # the state is exact fp32 in both, and every token runs the same arithmetic
    B, T, HK, HV, dk, dv = 3, 9, 2, 4, 128, 64
    x = small_inputs(B, T, HK, HV, dk, dv, seed=41)
    d = dev(x)
    note("recurrent vs successive decode steps, bitwise")
    o_f, ht_f = gdr.fused_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"])
    state = d["h0"].clone()
    o_s = torch.empty(B, T, HV, dv, device="cuda")
    for t in range(T):
        sl = {n: d[n][:, t:t + 1].contiguous() for n in ("q", "k", "v", "g", "beta")}
        o_t = gdr.decode_step(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], state)
        o_s[:, t:t + 1] = o_t
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_s)
    assert torch.equal(ht_f, state)


def test_recurrent_one_token_equals_decode_step_bitwise():
    x = small_inputs(4, 1, 2, 4, 128, 128, seed=43)
    d = dev(x)
    note("recurrent T=1 vs decode step, bitwise")
    o_f, ht_f = gdr.fused_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"])
    state = d["h0"].clone()
    o_d = gdr.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state)
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_d) and torch.equal(ht_f, state)


def test_recurrent_matches_chunked_prefill():
    x = small_inputs(2, 45, 2, 4, 128, 128, seed=47)
    d = dev(x)
    note("recurrent vs chunked prefill T=45")
    o_r, ht_r = gdr.fused_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"])
    o_c, ht_c = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=32)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.sequential(**x)
    assert err(o_r, o_ref) < TOL and err(o_c, o_ref) < TOL
    assert err(ht_r, ht_ref) < TOL and err(ht_c, ht_ref) < TOL


def test_recurrent_in_place_and_no_state_output():
    x = small_inputs(2, 5, 1, 2, 64, 64, seed=53)
    o_ref, ht_ref = oracle.sequential(**x)
    d = dev(x)
    note("recurrent in place (ht == h0), then ht not wanted")
    state = d["h0"].clone()
    o1, ht1 = gdr.fused_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=state, ht=state)
    o2, ht2 = gdr.fused_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], want_state=False)
    torch.cuda.synchronize()
    assert ht1.data_ptr() == state.data_ptr() and ht2 is None
    assert err(o1, o_ref) < TOL and err(state, ht_ref) < TOL
    assert torch.equal(o1, o2)


def test_recurrent_full_size_short_call_sampled():
    """A short call at the decode workload's size: B=32, HK=16, HV=32, dk=dv=128 and 16
    tokens (a speculative chain), with the decode workload's input recipe; sampled
    (batch, key-head) groups are checked against the oracle."""
    w = DECODE
    T = 16
    x = make_inputs(w.B, T, w.HK, w.HV, w.dk, w.dv, dtype=w.dtype, seed=w.seed + 1000, h0=True)
    d = dev(x)
    note("recurrent full size B=32 T=16")
    o, ht = gdr.fused_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"])
    torch.cuda.synchronize()
    G = w.HV // w.HK
    groups = sampled_groups(w.B, w.HK, 4, seed=3)
    ref = oracle_on_groups(x, groups, G)
    o_c, st = o.cpu(), ht.cpu()
    for (b, kh), (o_r, ht_r) in ref.items():
        hv = slice(kh * G, (kh + 1) * G)
        eo, es = err(o_c[b, :, hv], o_r), err(st[b, hv], ht_r)
        assert eo < TOL and es < TOL, f"group {(b, kh)}: o {eo:.2e} state {es:.2e}"


@pytest.mark.parametrize("T", [gdr.RECURRENT_MAX_T, gdr.RECURRENT_MAX_T + 1, 40])
def test_forward_routes_to_the_measured_path(T):
    x = small_inputs(2, T, 2, 4, 128, 128, seed=59 + T)
    o_ref, ht_ref = oracle.sequential(**x)
    d = dev(x)
    note(f"forward routing T={T}")
    o_f, ht_f = gdr.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=32)
    if T <= gdr.RECURRENT_MAX_T:
        o_p, ht_p = gdr.fused_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"])
    else:
        o_p, ht_p = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=32)
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_p) and torch.equal(ht_f, ht_p)
    assert err(o_f, o_ref) < TOL and err(ht_f, ht_ref) < TOL
