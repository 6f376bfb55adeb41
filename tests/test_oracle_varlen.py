"""Pins of the oracle's packed variable-length batch (oracle.varlen): sequences laid end to
end, each run from its own initial state (ExecuTorch PR #21021, second commit summary,
routes by sequence length; the batch format is this library's reading).

The pins: equal-length sequences packed give exactly the dense batch of the same rows;
permuting the sequences permutes the results; a sequence with no rows passes its h0 through;
a sequence's result does not depend on its neighbours; the chunked route agrees with the
sequential one.  Planted mistakes (a state carried across sequences, a slice one row short,
the wrong h0 row) are caught."""
import numpy as np
import pytest
import torch

import oracle
from gdr_synth import make_inputs


def _packed(lengths, seed=0, HK=2, HV=4, dk=8, dv=6, h0=True):
    T = sum(lengths)
    x = make_inputs(1, T, HK, HV, dk, dv, dtype=torch.float32, seed=seed, h0=False)
    x = {n: t[0].double().numpy() for n, t in x.items() if t is not None}
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rng = np.random.default_rng(seed + 1)
    x["h0"] = 0.3 * rng.standard_normal((len(lengths), HV, dk, dv)) if h0 else None
    return x, cu


def equal_length_pin(fn):
    B, T = 3, 7
    x, cu = _packed([T] * B, seed=2)
    o, ht = fn(x, cu)
    dense = {n: (x[n].reshape(B, T, *x[n].shape[1:]) if n != "h0" else x[n]) for n in x}
    od, htd = oracle.sequential(**dense)
    assert np.allclose(o.reshape(B, T, *o.shape[1:]), od, rtol=1e-13, atol=1e-14)
    assert np.allclose(ht, htd, rtol=1e-13, atol=1e-14)


def permutation_pin(fn):
    lengths = [5, 1, 9, 3]
    x, cu = _packed(lengths, seed=3)
    o, ht = fn(x, cu)
    order = [2, 0, 3, 1]
    rows = [np.arange(cu[i], cu[i + 1]) for i in order]
    idx = np.concatenate(rows)
    y = {n: (x[n][idx] if n != "h0" else x[n][order]) for n in x}
    cu2 = np.concatenate([[0], np.cumsum([lengths[i] for i in order])]).astype(np.int32)
    o2, ht2 = fn(y, cu2)
    assert np.allclose(o2, o[idx], rtol=1e-13, atol=1e-14)
    assert np.allclose(ht2, ht[order], rtol=1e-13, atol=1e-14)


def empty_sequence_pin(fn):
    x, cu = _packed([4, 0, 6], seed=4)
    o, ht = fn(x, cu)
    assert np.array_equal(ht[1], x["h0"][1])
    # neighbours unaffected: the same two sequences without the empty one
    y = dict(x, h0=x["h0"][[0, 2]])
    o2, ht2 = fn(y, np.array([0, 4, 10], np.int32))
    assert np.allclose(o2, o, rtol=1e-13, atol=1e-14) and np.allclose(ht2, ht[[0, 2]], rtol=1e-13, atol=1e-14)


def independence_pin(fn):
    lengths = [6, 5]
    x, cu = _packed(lengths, seed=5)
    o, ht = fn(x, cu)
    y = {n: x[n].copy() for n in x}
    y["v"][6:] *= -3.0  # change only the second sequence
    y["h0"][1] += 1.0
    o2, ht2 = fn(y, cu)
    assert np.array_equal(o2[:6], o[:6]) and np.array_equal(ht2[0], ht[0])
    assert not np.allclose(o2[6:], o[6:])


def all_pins(fn):
    equal_length_pin(fn)
    permutation_pin(fn)
    empty_sequence_pin(fn)
    independence_pin(fn)


def seq(x, cu):
    return oracle.varlen(oracle.sequential, cu_seqlens=cu, **x)


def test_varlen_pins():
    all_pins(seq)


def test_varlen_chunked_route_matches():
    x, cu = _packed([1, 15, 40, 33], seed=6)
    o1, h1 = seq(x, cu)
    o2, h2 = oracle.varlen(oracle.chunked, cu_seqlens=cu, chunk=16, **x)
    assert np.allclose(o2, o1, rtol=1e-11, atol=1e-12) and np.allclose(h2, h1, rtol=1e-11, atol=1e-12)


def _carry_across(x, cu):
    """Mistake: the state runs on from one sequence into the next."""
    o, _ = oracle.sequential(**{n: (x[n][None] if n != "h0" else (None if x["h0"] is None else x["h0"][:1]))
                                for n in x})
    o = o[0]
    ht = np.stack([oracle.sequential(**{n: (x[n][None, :cu[i + 1]] if n != "h0" else x["h0"][:1]) for n in x})[1][0]
                   for i in range(len(cu) - 1)])
    return o, ht


def _short_slice(x, cu):
    """Mistake: each sequence loses its last row."""
    N = len(cu) - 1
    T, HV, dv = x["v"].shape
    o = np.zeros((T, HV, dv))
    ht = np.zeros((N,) + x["h0"].shape[1:])
    for i in range(N):
        a, b = cu[i], max(cu[i], cu[i + 1] - 1)
        if b == a:
            ht[i] = x["h0"][i]
            continue
        oi, hi = oracle.sequential(**{n: (x[n][None, a:b] if n != "h0" else x["h0"][i:i + 1]) for n in x})
        o[a:b] = oi[0]
        ht[i] = hi[0]
    return o, ht


def _shifted_h0(x, cu):
    """Mistake: sequence i starts from the h0 row of sequence i + 1."""
    return seq(dict(x, h0=np.roll(x["h0"], -1, axis=0)), cu)


MUTANTS = {"carry_across": _carry_across, "short_slice": _short_slice, "shifted_h0": _shifted_h0}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_varlen_mutants_are_caught(name):
    with pytest.raises(AssertionError):
        all_pins(MUTANTS[name])
