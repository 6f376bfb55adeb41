"""The chunked prefill over the input range: the recurrence is linear in (h0, v) jointly
and o is linear in q, so a copy of a passing case scaled by a power of two is an equally
valid input and must pass the same bar against the fp64 oracle (run on the scaled
inputs, which bf16 and fp32 represent exactly).  Every carry form is exercised: the
column split with 4, 2 and 1 waves per workgroup (chunk 64, 32, 16) and with four column
tiles per workgroup (96 heads), one workgroup per head (more than 128 heads) and the
time-segmented carry (few heads, many chunks)."""
import zlib

import pytest
import torch

import gated_delta_rule_70_amd as gdr
import oracle
from gpu_util import TOL, dev, err, note, small_inputs

pytestmark = pytest.mark.gpu

# (B, T, HK, HV, dk, dv, chunk)
CASES = {
    "split_c64": (2, 200, 2, 4, 128, 128, 64),
    "split_c32": (2, 200, 2, 4, 128, 128, 32),
    "split_c16": (2, 120, 2, 4, 64, 64, 16),
    "split_4_tiles": (3, 130, 16, 32, 128, 128, 64),
    "whole_head": (2, 150, 40, 80, 128, 128, 64),
    "segmented": (2, 4100, 16, 32, 64, 64, 64),
}
SCALES = {
    "vh_up": {"v": 2.0 ** 14, "h0": 2.0 ** 14},
    "vh_down": {"v": 2.0 ** -18, "h0": 2.0 ** -18},
    "q_up": {"q": 2.0 ** 10},
    "q_down": {"q": 2.0 ** -20},
    "h0_up": {"h0": 2.0 ** 12},
    "v_down": {"v": 2.0 ** -12},
}


def _scaled(case, scale, dtype, seed):
    B, T, HK, HV, dk, dv, C = CASES[case]
    x = small_inputs(B, T, HK, HV, dk, dv, dtype=dtype, seed=seed)
    for name, f in SCALES[scale].items():
        x[name] = (x[name].double() * f).to(x[name].dtype)
    return x, C


def _route(case):
    """The carry form the library picks for this case, from the workspace it asks for."""
    B, T, HK, HV, dk, dv, C = CASES[case]
    need = gdr.workspace_bytes(B, T, HK, HV, dk, dv, C)
    nc = -(-T // C)
    rec = need if need == B * HV * nc * (gdr.workspace_bytes(1, C, 1, 1, dk, dv, C)) else None
    return "segmented" if rec is None else "records only"


@pytest.mark.parametrize("scale", sorted(SCALES))
@pytest.mark.parametrize("case", sorted(CASES))
def test_scaled_inputs_bf16(case, scale):
    x, C = _scaled(case, scale, torch.bfloat16, seed=zlib.crc32(f"{case}/{scale}".encode()) % 1000)
    assert (_route(case) == "segmented") == (case == "segmented")
    o_ref, ht_ref = oracle.sequential(**x)
    note(f"range {case} {scale} bf16")
    d = dev(x)
    o, ht = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C)
    torch.cuda.synchronize()
    eo, es = err(o, o_ref), err(ht, ht_ref)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


@pytest.mark.parametrize("scale", ["vh_up", "vh_down", "q_down", "h0_up"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_scaled_inputs_fp32(case, scale):
    x, C = _scaled(case, scale, torch.float32, seed=7 + zlib.crc32(f"{case}/{scale}".encode()) % 1000)
    o_ref, ht_ref = oracle.sequential(**x)
    note(f"range {case} {scale} fp32")
    d = dev(x)
    o, ht = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C)
    torch.cuda.synchronize()
    eo, es = err(o, o_ref), err(ht, ht_ref)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"


@pytest.mark.parametrize("case", ["split_c64", "whole_head"])
def test_zero_initial_state_with_tiny_v(case):
    """h0 = NULL and v scaled by 2^-24: the state starts at exactly zero and takes its
    scale from v alone."""
    x, C = _scaled(case, "vh_down", torch.bfloat16, seed=11)
    x["v"] = (x["v"].double() * 2.0 ** -6).to(torch.bfloat16)
    x["h0"] = None
    o_ref, ht_ref = oracle.sequential(**x)
    note(f"range {case} zero h0, v * 2^-24")
    d = dev(x)
    o, ht = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=None, chunk=C)
    torch.cuda.synchronize()
    eo, es = err(o, o_ref), err(ht, ht_ref)
    assert eo < TOL and es < TOL, f"o {eo:.2e} state {es:.2e}"
