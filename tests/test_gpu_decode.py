"""Decode step (T == 1) on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

import gated_delta_rule_70_amd as gdr
import oracle
from gdr_synth import DECODE, workload_inputs
from gpu_util import TOL, bf16_exact_unit_keys, dev, err, note, small_inputs

pytestmark = pytest.mark.gpu

DIMS = [(32, 32), (32, 128), (64, 64), (128, 32), (128, 64), (128, 128), (64, 128)]


@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("G", [1, 2])
@pytest.mark.parametrize("h0", [True, False])
def test_decode_one_step(dk, dv, dtype, G, h0):
    x = small_inputs(3, 1, 2, 2 * G, dk, dv, dtype=dtype, seed=dk + dv + G, h0=h0)
    o_ref, ht_ref = oracle.sequential(**x)
    d = dev(x)
    state = d["h0"].clone() if h0 else None
    out_state = None if h0 else torch.full((3, 2 * G, dk, dv), float("nan"), device="cuda")
    note(f"decode one step dk={dk} dv={dv} {dtype} G={G} h0={h0}")
    o = gdr.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, out_state=out_state)
    torch.cuda.synchronize()
    new_state = state if h0 else out_state
    assert err(o, o_ref) < TOL and err(new_state, ht_ref) < TOL


def _step_views(x):
    """Per-step contiguous views [B,1,H,d] of inputs drawn as [B,T,H,d]."""
    T = x["q"].shape[1]
    tm = {n: x[n].transpose(0, 1).contiguous() for n in ("q", "k", "v", "g", "beta")}
    return T, tm


def _run_steps(d, state, T, tm, obuf):
    for t in range(T):
        o_t = obuf[t].unsqueeze(1)
        gdr.decode_step(tm["q"][t].unsqueeze(1), tm["k"][t].unsqueeze(1), tm["v"][t].unsqueeze(1),
                        tm["g"][t].unsqueeze(1), tm["beta"][t].unsqueeze(1), state, o=o_t)


def test_decode_many_steps_in_place():
    x = small_inputs(2, 37, 2, 4, 128, 128, seed=5)
    o_ref, ht_ref = oracle.sequential(**x)
    d = dev(x)
    T, tm = _step_views(d)
    state = d["h0"].clone()
    obuf = torch.empty(T, 2, 4, 128, device="cuda")
    note("decode 37 carried steps")
    _run_steps(d, state, T, tm, obuf)
    torch.cuda.synchronize()
    assert err(obuf.transpose(0, 1), o_ref) < TOL and err(state, ht_ref) < TOL


def test_decode_full_size_1000_steps_all_heads():
    """The measured decode workload: B=32, HK=16, HV=32, dk=dv=128, 1000 carried steps,
    every (batch, value head) checked against the oracle on all 1000 outputs and on the
    final state."""
    w = DECODE
    x = workload_inputs(w)
    d = dev(x)
    T, tm = _step_views(d)
    state = d["h0"].clone()
    obuf = torch.empty(T, w.B, w.HV, w.dv, device="cuda")
    note("decode full size 1000 steps")
    _run_steps(d, state, T, tm, obuf)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.sequential(**x)
    eo = err(obuf.transpose(0, 1), o_ref)
    es = err(state, ht_ref)
    print(f"decode 1000 steps: o {eo:.2e} state {es:.2e}")
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


def test_decode_exact_write():
    # beta = 1, unit keys exact in bf16, q = k: the output equals v after any decay/state
    B, HK, HV, dk, dv = 4, 2, 4, 128, 64
    x = small_inputs(B, 1, HK, HV, dk, dv, seed=9)
    k = bf16_exact_unit_keys(B, 1, HK, dk, seed=3).to(torch.bfloat16)
    x["k"] = k
    x["q"] = k.clone()
    x["beta"] = torch.ones_like(x["beta"])
    d = dev(x)
    note("decode exact write")
    o = gdr.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"].clone())
    torch.cuda.synchronize()
    v = x["v"].float()
    assert float((o.cpu() - v).abs().max()) < 1e-5 * float(v.abs().max()) + 1e-6


def test_decode_equals_prefill_one_token():
    x = small_inputs(2, 1, 2, 4, 128, 128, seed=13)
    d = dev(x)
    note("decode vs prefill T=1")
    o1 = gdr.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"].clone())
    o2, _ = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=64)
    torch.cuda.synchronize()
    o_ref, _ = oracle.sequential(**x)
    assert err(o1, o_ref) < TOL and err(o2, o_ref) < TOL
    assert err(o1, o2.double().cpu().numpy()) < TOL


def test_decode_deterministic():
    x = small_inputs(8, 1, 4, 8, 128, 128, seed=17)
    d = dev(x)
    note("decode determinism")
    s1, s2 = d["h0"].clone(), d["h0"].clone()
    o1 = gdr.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], s1)
    o2 = gdr.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
