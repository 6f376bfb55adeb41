"""Host-only checks of the Python binding: every tensor's shape is compared with the dims
taken from q and v before any pointer is passed to the library (the C ABI cannot see
allocation sizes).  CPU tensors suffice: the shape check runs first and raises before the
device checks, so no kernel is launched and no GPU is needed."""
import pytest
import torch

import gated_delta_rule_70_amd as gdr

B, T, HK, HV, DK, DV = 2, 5, 2, 4, 32, 64


def good():
    return dict(q=torch.zeros(B, T, HK, DK), k=torch.zeros(B, T, HK, DK), v=torch.zeros(B, T, HV, DV),
                g=torch.zeros(B, T, HV, DK), beta=torch.zeros(B, T, HV))


BAD = {
    "k": torch.zeros(B, T, HK, DK + 1),
    "v": torch.zeros(B, T - 1, HV, DV),
    "g_wrong_heads": torch.zeros(B, T, HK + 1, DK),
    "beta_per_key_head": torch.zeros(B, T, HK),
}


def _name(case):
    return case.split("_")[0]


@pytest.mark.parametrize("case", sorted(BAD))
@pytest.mark.parametrize("entry", ["chunk_prefill", "fused_recurrent", "forward", "decode_step", "tree_verify"])
def test_input_shape_mismatch_raises(case, entry):
    x = good()
    x[_name(case)] = BAD[case]
    T1 = 1 if entry == "decode_step" else T
    if entry == "decode_step":
        x = {n: t[:, :1].contiguous() if t.shape[1] == T else t for n, t in x.items()}
        x[_name(case)] = BAD[case][:, :1] if BAD[case].shape[1] == T else BAD[case]
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"])
    with pytest.raises(ValueError, match=rf"^{_name(case)} must"):
        if entry == "decode_step":
            gdr.decode_step(*args, torch.zeros(B, HV, DK, DV))
        elif entry == "tree_verify":
            gdr.tree_verify(*args, parent=torch.zeros(B, T1, dtype=torch.int32))
        else:
            getattr(gdr, entry)(*args)


@pytest.mark.parametrize("what,shape", [
    ("h0", (B, HV, DK, DK)), ("h0", (B, HK, DK, DV)), ("o", (B, T, HV, DV // 2)),
    ("ht", (B, HV, DV, DK)), ("o", (B, T, HK, DV))])
def test_state_and_output_shape_mismatch_raises(what, shape):
    x = good()
    bad = torch.zeros(*shape)
    with pytest.raises(ValueError, match=rf"^{what} must"):
        gdr.chunk_prefill(**x, **{what: bad})
    with pytest.raises(ValueError, match=rf"^{what} must"):
        gdr.fused_recurrent(**x, **{what: bad})


def test_decode_state_shape_mismatch_raises():
    x = {n: t[:, :1].contiguous() for n, t in good().items()}
    with pytest.raises(ValueError, match=r"^h0 must"):
        gdr.decode_step(**x, state=torch.zeros(B, HV, DK, DV + 16))
    with pytest.raises(ValueError, match=r"^ht must"):
        gdr.decode_step(**x, state=None, out_state=torch.zeros(B, HV, DK))


def test_tree_parent_shape_mismatch_raises():
    with pytest.raises(ValueError, match=r"^parent must"):
        gdr.tree_verify(**good(), parent=torch.zeros(B, T + 1, dtype=torch.int32))


def test_well_shaped_cpu_tensors_fail_only_on_device():
    # the shape check passes; the next check (device) is what rejects CPU tensors
    with pytest.raises(ValueError, match="GPU tensor"):
        gdr.chunk_prefill(**good(), h0=torch.zeros(B, HV, DK, DV))


def test_key_head_gate_shape_is_accepted():
    # g [B,T,HK,dk] (a gate per key head) passes the shape check on every entry point
    x = good()
    x["g"] = torch.zeros(B, T, HK, DK)
    for entry in ("chunk_prefill", "fused_recurrent", "forward"):
        with pytest.raises(ValueError, match="GPU tensor"):
            getattr(gdr, entry)(**x)
