"""The oracle's chunkwise WY/UT route against its token recurrence and closed forms.

The chunked form is an exact rewrite of the recurrence (second commit summary of
ExecuTorch PR #21021), so the two fp64 routes must agree to rounding for every chunk
size, ragged length, head grouping and initial state.
"""
import numpy as np
import pytest

import oracle
from oracle_pins import random_inputs, rel

TIGHT = 1e-11


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 15, 17, 33, 64, 97])
@pytest.mark.parametrize("G", [1, 2])
@pytest.mark.parametrize("h0", [False, True])
def test_chunked_equals_sequential(C, T, G, h0):
    x = random_inputs(100 + T + C + G, B=2, T=T, HK=2, HV=2 * G, dk=8, dv=6, h0=h0)
    o_s, ht_s = oracle.sequential(**x)
    o_c, ht_c = oracle.chunked(**x, chunk=C)
    assert rel(o_c, o_s) < TIGHT and rel(ht_c, ht_s) < TIGHT


@pytest.mark.parametrize("T", [64, 97])
def test_chunk_size_invariance_real_magnitudes(T):
    # dk = dv = 32, softplus decays, unit keys: the regime the GPU path runs in
    x = random_inputs(7 + T, B=1, T=T, HK=1, HV=2, dk=32, dv=32, h0=True)
    outs = [oracle.chunked(**x, chunk=C) for C in (1, 16, 32, 64)]
    for o, ht in outs[1:]:
        assert rel(o, outs[0][0]) < TIGHT and rel(ht, outs[0][1]) < TIGHT


def test_intermediates_scalar_gate_closed_form():
    # P11: a gate constant across channels gives A_rs = beta_r exp(gam_r - gam_s) (k_r . k_s)
    # and P_rs = exp(gam_r - gam_s) (q_r . k_s), gam the inclusive prefix of the scalar gate.
    x = random_inputs(31, B=1, T=21, HK=1, HV=1, dk=5, dv=4)
    scal = x["g"][..., :1]
    x["g"] = np.repeat(scal, 5, axis=-1)
    C = 8
    _, _, mids = oracle.chunked(**x, chunk=C, intermediates=True)
    err = 0.0
    for n in range(3):
        t0 = n * C
        L = min(C, 21 - t0)
        gam = np.cumsum(scal[0, t0:t0 + L, 0, 0])
        kk = x["k"][0, t0:t0 + L, 0]
        qq = x["q"][0, t0:t0 + L, 0]
        bb = x["beta"][0, t0:t0 + L, 0]
        dec = np.exp(gam[:, None] - gam[None, :])
        A_ref = np.tril(bb[:, None] * dec * (kk @ kk.T), -1)
        P_ref = np.tril(dec * (qq @ kk.T))
        err = max(err, np.max(np.abs(mids["A"][0, 0, n, :L, :L] - A_ref)),
                  np.max(np.abs(mids["P"][0, 0, n, :L, :L] - P_ref)))
    assert err < 1e-12


def test_intermediates_solve_and_carry():
    # W and Ubar solve (I + A) X = [diag(beta) exp(gam) k | diag(beta) v]; check with a
    # dense library solve, and U = Ubar - W S0 with S0 the sequential state at chunk start.
    x = random_inputs(32, B=1, T=40, HK=1, HV=1, dk=6, dv=5, h0=True)
    C = 16
    _, _, mids = oracle.chunked(**x, chunk=C, intermediates=True)
    err = 0.0
    for n in range(3):
        t0 = n * C
        L = min(C, 40 - t0)
        A = mids["A"][0, 0, n, :L, :L]
        gam = np.cumsum(x["g"][0, t0:t0 + L, 0], axis=0)
        bb = x["beta"][0, t0:t0 + L, 0]
        rhs = np.concatenate([bb[:, None] * np.exp(gam) * x["k"][0, t0:t0 + L, 0],
                              bb[:, None] * x["v"][0, t0:t0 + L, 0]], axis=1)
        X = np.linalg.solve(np.eye(L) + A, rhs)
        err = max(err, np.max(np.abs(mids["W"][0, 0, n, :L] - X[:, :6])),
                  np.max(np.abs(mids["Ubar"][0, 0, n, :L] - X[:, 6:])))
        if t0 == 0:
            S0 = x["h0"][0, 0]
        else:
            sub = {k: (a[:, :t0] if k != "h0" else a) for k, a in x.items()}
            S0 = oracle.sequential(**sub)[1][0, 0]
        err = max(err, np.max(np.abs(mids["U"][0, 0, n, :L] - (X[:, 6:] - X[:, :6] @ S0))))
        # the last chunk's rows past L are zero in every export
        assert np.all(mids["W"][0, 0, n, L:] == 0)
    assert err < 1e-11
