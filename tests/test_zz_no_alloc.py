"""The allocation-free prefill entry point (gdr_chunk_prefill_noalloc, through the C ABI)
against the existing one (gdr_chunk_prefill with a caller workspace): two calls in a row,
the second smaller, each equal bit for bit to the existing entry point's result and within
the parity bar of the fp64 oracle; and a call needing more than the scratch is refused on
the host."""
import pytest
import torch

import gated_delta_rule_70_amd as gdr
import oracle
from gpu_util import TOL, dev, err, note, small_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cases", [[(2, 300, 2, 4, 128, 128, 64), (1, 77, 2, 4, 128, 128, 64)],
                                   [(2, 150, 40, 80, 128, 128, 64), (1, 33, 1, 2, 64, 64, 16)]],
                         ids=["column_split", "whole_head_then_small"])
def test_noalloc_matches_prefill_twice(cases):
    for i, (B, T, HK, HV, dk, dv, C) in enumerate(cases):
        x = small_inputs(B, T, HK, HV, dk, dv, seed=500 + i)
        d = dev(x)
        assert gdr.workspace_bytes(B, T, HK, HV, dk, dv, C) <= gdr.NOALLOC_SCRATCH_BYTES
        note(f"noalloc prefill call {i}: B={B} T={T} HV={HV} dk={dk} C={C}")
        o_ref_gpu, ht_ref_gpu = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C)
        o = torch.full_like(o_ref_gpu, float("nan"))
        ht = torch.full_like(ht_ref_gpu, float("nan"))
        gdr.chunk_prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C, o=o, ht=ht)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref_gpu) and torch.equal(ht, ht_ref_gpu)
        o_ref, ht_ref = oracle.sequential(**x)
        assert err(o, o_ref) < TOL and err(ht, ht_ref) < TOL


def test_noalloc_refuses_calls_past_its_scratch():
    B, T, HK, HV, dk, dv, C = 1, 4097, 16, 32, 128, 128, 64
    assert gdr.workspace_bytes(B, T, HK, HV, dk, dv, C) > gdr.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, T, HK, dk, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(B, T, HV, dv, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(B, T, HV, dk, device="cuda")
    beta = torch.zeros(B, T, HV, device="cuda")
    note("noalloc refusal")
    with pytest.raises(gdr.GdrError) as e:
        gdr.chunk_prefill_noalloc(q, q, v, g, beta, chunk=C)
    assert e.value.status == 8
