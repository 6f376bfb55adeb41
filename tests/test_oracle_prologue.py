"""Pins of the oracle's input pre-processing (the fused prologue's reference): the softplus
decay against scipy's log-sigmoid and its closed forms, the key normalisation against its
defining properties; planted mistakes in either are caught."""
import numpy as np
import pytest
from scipy.special import log_expit

import oracle


def softplus_pins(ns):
    a = np.linspace(-30.0, 30.0, 2001)
    # -softplus(a) = log(sigmoid(-a)), a library routine
    assert np.allclose(ns(a), log_expit(-a), rtol=1e-14, atol=1e-300)
    # softplus(a) - softplus(-a) = a;  softplus(0) = ln 2
    assert np.allclose(ns(-a) - ns(a), a, rtol=0, atol=1e-12)
    assert ns(np.array([0.0]))[0] == pytest.approx(-np.log(2.0), rel=1e-15)
    # tails: -softplus(a) -> -a - e^-a for large a, -> -e^a for very negative a (no cancellation)
    assert ns(np.array([40.0]))[0] == pytest.approx(-40.0 - np.exp(-40.0), rel=1e-15)
    assert ns(np.array([-40.0]))[0] == pytest.approx(-np.exp(-40.0), rel=1e-12)
    assert ns(np.array([800.0]))[0] == -800.0 and ns(np.array([-800.0]))[0] == -0.0


def l2norm_pins(nk):
    rng = np.random.default_rng(5)
    k = rng.standard_normal((3, 7, 2, 32)) * rng.uniform(0.01, 100.0, (3, 7, 2, 1))
    kh = nk(k)
    # unit norm per token and head, same direction, scale invariant, zero stays zero
    assert np.allclose(np.linalg.norm(kh, axis=-1), 1.0, rtol=1e-14)
    assert np.allclose(np.sum(kh * k, axis=-1), np.sqrt(np.sum(k * k, axis=-1)), rtol=1e-13)
    assert np.allclose(nk(7.25 * k), kh, rtol=1e-14, atol=0)
    z = np.zeros((1, 1, 1, 32))
    assert np.array_equal(nk(z), z)


def test_neg_softplus_pins():
    softplus_pins(oracle.neg_softplus)


def test_l2_normalize_keys_pins():
    l2norm_pins(oracle.l2_normalize_keys)


MUTANTS = {
    "softplus of -a": lambda a: -(np.maximum(-a, 0.0) + np.log1p(np.exp(-np.abs(a)))),
    "no log1p term": lambda a: -np.maximum(a, 0.0),
    "wrong sign": lambda a: np.maximum(a, 0.0) + np.log1p(np.exp(-np.abs(a))),
    "log instead of log1p": lambda a: -(np.maximum(a, 0.0) + np.log(np.exp(-np.abs(a)))),
}
KEY_MUTANTS = {
    "norm over heads": lambda k: k / np.sqrt(np.sum(k * k, axis=-2, keepdims=True)),
    "squared norm": lambda k: k / np.sum(k * k, axis=-1, keepdims=True),
    "max-norm": lambda k: k / np.max(np.abs(k), axis=-1, keepdims=True),
    "no eps (zero keys)": lambda k: k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_softplus_mutants_are_caught(name):
    with pytest.raises(AssertionError):
        softplus_pins(MUTANTS[name])


@pytest.mark.parametrize("name", sorted(KEY_MUTANTS))
def test_key_norm_mutants_are_caught(name):
    with np.errstate(all="ignore"):
        with pytest.raises(AssertionError):
            l2norm_pins(KEY_MUTANTS[name])
