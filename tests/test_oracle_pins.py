"""The fp64 oracle against hand-worked values, closed forms, brute force and invariants."""
import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS, TOL, brute_force, random_inputs, rel

ROUTES = [("sequential", None), ("chunked", 1), ("chunked", 2), ("chunked", 3), ("chunked", 16)]


@pytest.mark.parametrize("name", sorted(ALL_PINS))
@pytest.mark.parametrize("route,chunk", ROUTES)
def test_pin(name, route, chunk):
    lib = oracle.load()
    kw = {} if chunk is None else {"chunk": chunk}
    if name == "scalar_gate_gram" and route == "sequential":
        pytest.skip("intermediates exist only on the chunked route")
    err = ALL_PINS[name](lib, route=route, **kw)
    assert err < TOL, f"{name} via {route}(chunk={chunk}): error {err:.3e}"


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_brute_force_gqa_shapes(seed):
    # dk != dv and G = 3 so that a transposed state or a wrong head map cannot hide
    x = random_inputs(seed, B=1, T=5, HK=2, HV=6, dk=3, dv=5)
    o, ht = oracle.sequential(**x)
    o_ref, ht_ref = brute_force(x)
    assert rel(o, o_ref) < TOL and rel(ht, ht_ref) < TOL


def test_no_initial_state_equals_zero_state():
    x = random_inputs(24, B=1, T=6, HK=1, HV=2, dk=4, dv=4)
    o1, ht1 = oracle.sequential(**dict(x, h0=None))
    o2, ht2 = oracle.sequential(**dict(x, h0=np.zeros_like(x["h0"])))
    assert np.array_equal(o1, o2) and np.array_equal(ht1, ht2)


def test_thread_count_does_not_change_results():
    x = random_inputs(25, B=3, T=20, HK=2, HV=4, dk=8, dv=8)
    o1, ht1 = oracle.sequential(**x, threads=1)
    o2, ht2 = oracle.sequential(**x, threads=4)
    assert np.array_equal(o1, o2) and np.array_equal(ht1, ht2)


def test_rejects_bad_shapes():
    x = random_inputs(26, B=1, T=3, HK=2, HV=3, dk=2, dv=2)
    with pytest.raises(ValueError):
        oracle.sequential(**x)
