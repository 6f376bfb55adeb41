"""Pins of the oracle's gate shared per key head (g ``[B,T,HK,dk]``, beta per value head):
every value head of a GQA group decays with its key head's gate, h -> h // G, the layout
that the uzu PR #576 review thread on the per-value-head gram weighs against a gate per
value head.

The pins: each value head's result equals a single-head oracle run on that head's own
slices (key head h // G for q, k and g), on the sequential, chunked and tree routes; value
heads of one group given the same beta, v and h0 give identical results; the expansion
itself matches the head map written out index by index.  A wrong head map (h % HK, or the
gate of the first group for every head) is caught."""
import numpy as np
import torch
import pytest

import oracle
from gdr_synth import make_inputs, make_tree


def _inputs(seed=3, B=2, T=11, HK=3, HV=6, dk=8, dv=5):
    return {n: (None if t is None else t.double().numpy())
            for n, t in make_inputs(B, T, HK, HV, dk, dv, dtype=torch.float32,
                                    seed=seed, h0=True, gate_heads="key").items()}


def _per_head(x, h, G):
    kh = h // G
    return dict(q=x["q"][:, :, kh:kh + 1], k=x["k"][:, :, kh:kh + 1], v=x["v"][:, :, h:h + 1],
                g=x["g"][:, :, kh:kh + 1], beta=x["beta"][:, :, h:h + 1], h0=x["h0"][:, h:h + 1])


def per_head_pin(expand, route):
    """Value head h of the grouped call == a one-head call on its own slices."""
    x = _inputs()
    HK, HV = x["q"].shape[2], x["v"].shape[2]
    G = HV // HK
    full = dict(x, g=expand(x["g"], HV))
    par = np.asarray(make_tree(2, 11, "random", seed=4))
    run = {
        "sequential": lambda a: oracle.sequential(**a),
        "chunked": lambda a: oracle.chunked(**a, chunk=4),
        "tree": lambda a: (oracle.tree(**a, parent=par), None),
    }[route]
    o, ht = run(full)
    for h in range(HV):
        oh, hth = run(_per_head(x, h, G))
        assert np.allclose(o[:, :, h:h + 1], oh, rtol=1e-12, atol=1e-14), f"o of value head {h}"
        if ht is not None:
            assert np.allclose(ht[:, h:h + 1], hth, rtol=1e-12, atol=1e-14), f"state of value head {h}"


def same_group_pin(expand):
    """With beta, v and h0 equal across a group, the group's value heads agree exactly; the
    groups differ from one another."""
    x = _inputs(seed=8)
    HK, HV = x["q"].shape[2], x["v"].shape[2]
    G = HV // HK
    for n in ("v", "beta"):
        x[n] = np.repeat(x[n][:, :, ::G], G, axis=2)
    x["h0"] = np.repeat(x["h0"][:, ::G], G, axis=1)
    o, ht = oracle.sequential(**dict(x, g=expand(x["g"], HV)))
    for h in range(HV):
        base = (h // G) * G
        assert np.array_equal(o[:, :, h], o[:, :, base]) and np.array_equal(ht[:, h], ht[:, base])
    assert not np.allclose(o[:, :, 0], o[:, :, G])


def index_pin(expand):
    x = _inputs(seed=9)
    HK, HV = x["g"].shape[2], x["v"].shape[2]
    e = expand(x["g"], HV)
    for h in range(HV):
        assert np.array_equal(e[:, :, h], x["g"][:, :, h // (HV // HK)])


def all_pins(expand):
    for route in ("sequential", "chunked", "tree"):
        per_head_pin(expand, route)
    same_group_pin(expand)
    index_pin(expand)


def test_gate_per_value_head_pins():
    all_pins(oracle.gate_per_value_head)


def test_routes_accept_key_head_gate_directly():
    """The routes expand a per-key-head gate themselves: the same result as expanding first."""
    x = _inputs(seed=12)
    HV = x["v"].shape[2]
    o1, h1 = oracle.sequential(**x)
    o2, h2 = oracle.sequential(**dict(x, g=oracle.gate_per_value_head(x["g"], HV)))
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)
    o3, h3 = oracle.chunked(**x, chunk=4)
    assert np.allclose(o3, o1, rtol=1e-12, atol=1e-13) and np.allclose(h3, h1, rtol=1e-12, atol=1e-13)


MUTANTS = {
    "h % HK": lambda g, HV: g[:, :, [h % g.shape[2] for h in range(HV)]],
    "first group only": lambda g, HV: np.repeat(g[:, :, :1], HV, axis=2),
    "tiled, not repeated": lambda g, HV: np.tile(g, (1, 1, HV // g.shape[2], 1)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_gate_head_mutants_are_caught(name):
    with pytest.raises(AssertionError):
        all_pins(MUTANTS[name])
