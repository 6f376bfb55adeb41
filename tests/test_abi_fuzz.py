"""Property-based checks of the host-side validation of libgdr.so (hypothesis), with fake
device addresses on a machine without a GPU: whatever the dims, flags, sizes and entry point,
a call returns one of the documented status codes without crashing, never reaches the HIP
runtime unless the workspace query accepts the same dims, and a call that does reach it is
refused on the host once its workspace is one byte short or misaligned."""
import ctypes

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import gated_delta_rule_70_amd as gdr
from test_abi import EHIP, EWS, OK, _gpu_visible, addr

STATUSES = set(range(9))
HEAD = [0, 16, 32, 48, 64, 128, 256]
CHUNK = [0, 8, 16, 32, 64, 128]
FLAG_BITS = [0, 1, 2, 3, 4, 5, 6, 12, 30]

# counting devices does not initialise the GPU
pytestmark = pytest.mark.skipif(_gpu_visible(), reason="valid fake pointers would reach a real GPU")


@pytest.fixture(scope="module")
def L():
    return gdr.lib()


def make_dims(B, T, HK, HV, dk, dv, chunk, dtype, flags):
    return gdr.Dims(B, T, HK, HV, dk, dv, chunk, dtype, flags)


def _valid_dims(B, T, HK, G, dk, dv, chunk, dtype, flags):
    return gdr.Dims(B, T, HK, HK * G, dk, dv, chunk, dtype, flags)


# shapes every check accepts (so the calls reach the runtime) ...
valid_dims = st.builds(
    _valid_dims,
    B=st.integers(1, 16), T=st.one_of(st.integers(1, 300), st.integers(100000, 300000)),
    HK=st.sampled_from([1, 2, 4, 8, 16]), G=st.sampled_from([1, 2, 4]),
    dk=st.sampled_from([32, 64, 128]), dv=st.sampled_from([32, 64, 128]), chunk=st.sampled_from([16, 32, 64]),
    dtype=st.just(0),
    flags=st.sampled_from([0, gdr.G_BF16, gdr.G_PER_KEY_HEAD, gdr.K_L2NORM | gdr.G_SOFTPLUS,
                           gdr.G_PER_KEY_HEAD | gdr.PREP_SPLIT, gdr.G_PER_KEY_HEAD | gdr.PREP_FUSED]),
)
# ... and anything at all
random_dims = st.builds(
    make_dims,
    B=st.integers(-1, 40), T=st.one_of(st.integers(-1, 300), st.integers(100000, 400000)),
    HK=st.integers(0, 20), HV=st.integers(0, 40),
    dk=st.sampled_from(HEAD), dv=st.sampled_from(HEAD), chunk=st.sampled_from(CHUNK),
    dtype=st.integers(0, 2),
    flags=st.lists(st.sampled_from(FLAG_BITS), max_size=3).map(lambda bits: sum({1 << b for b in bits})),
)
dims_strategy = st.one_of(valid_dims, random_dims)

PTRS = ["q", "k", "v", "g", "beta", "h0", "o", "ht", "ws"]


def call_prefill(L, entry, d, ws_bytes, ws=None):
    # tensors 2^40 bytes apart, so no two ranges overlap whatever the dims
    p = {n: ctypes.c_void_p((1 << 44) + i * (1 << 40)) for i, n in enumerate(PTRS)}
    if ws is not None:
        p["ws"] = ws
    return getattr(L, entry)(ctypes.byref(d), p["q"], p["k"], p["v"], p["g"], p["beta"], p["h0"], p["o"],
                             p["ht"], p["ws"], ctypes.c_size_t(ws_bytes), None)


@settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(d=dims_strategy, entry=st.sampled_from(["gdr_chunk_prefill", "gdr_chunk_prep", "gdr_chunk_carry", "gdr_forward"]))
def test_prefill_entries_validate_consistently(L, d, entry):
    need = int(L.gdr_chunk_prefill_workspace_bytes(ctypes.byref(d)))
    st_ = call_prefill(L, entry, d, need)
    assert st_ in STATUSES
    assert st_ != OK  # no GPU here: a call that passes every check fails at its first HIP call
    if need == 0 and entry != "gdr_forward":  # the token path of gdr_forward needs no workspace
        assert st_ != EHIP, "dims the workspace query rejects reached the runtime"
    if st_ == EHIP and need > 0:
        assert need % 256 == 0
        assert call_prefill(L, entry, d, need - 1) in (EWS, EHIP if entry == "gdr_forward" else EWS)
        assert call_prefill(L, entry, d, need, ws=ctypes.c_void_p((1 << 44) + 8 * (1 << 40) + 128)) in (
            EWS, EHIP if entry == "gdr_forward" else EWS)


@settings(max_examples=300, deadline=None)
@given(d=dims_strategy, entry=st.sampled_from(["gdr_decode_step", "gdr_fused_recurrent"]),
       misalign=st.sampled_from([0, 0, 0, 4, 8]))
def test_token_entries_validate_consistently(L, d, entry, misalign):
    p = {n: addr(i) for i, n in enumerate(["q", "k", "v", "g", "beta", "h0", "o", "ht"])}
    if misalign:
        p["v"] = addr(2, misalign)
    st_ = getattr(L, entry)(ctypes.byref(d), p["q"], p["k"], p["v"], p["g"], p["beta"], p["h0"], p["o"], p["ht"], None)
    assert st_ in STATUSES and st_ != OK
    if misalign:
        assert st_ != EHIP  # a misaligned tensor never reaches the runtime
    if entry == "gdr_decode_step" and d.T != 1:
        assert st_ != EHIP


@settings(max_examples=200, deadline=None)
@given(d=dims_strategy)
def test_packed_entries_validate_consistently(L, d):
    need = int(L.gdr_chunk_prefill_varlen_workspace_bytes(ctypes.byref(d)))
    p = {n: ctypes.c_void_p((1 << 44) + i * (1 << 40)) for i, n in enumerate(PTRS + ["cu"])}
    st_ = L.gdr_chunk_prefill_varlen(ctypes.byref(d), p["cu"], p["q"], p["k"], p["v"], p["g"], p["beta"], p["h0"],
                                     p["o"], p["ht"], p["ws"], ctypes.c_size_t(need), None)
    assert st_ in STATUSES and st_ != OK
    if need == 0:
        assert st_ != EHIP
    st2 = L.gdr_fused_recurrent_varlen(ctypes.byref(d), p["cu"], p["q"], p["k"], p["v"], p["g"], p["beta"], p["h0"],
                                       p["o"], p["ht"], None)
    assert st2 in STATUSES and st2 != OK
