"""Pins for the fp64 oracle: each returns an error that must be ~0 for a correct oracle.

Every pin checks the oracle against something other than itself: a hand-worked example,
a closed form, brute force with dense matrices, or an invariant of the mathematics.
They are written so that a plausible slip in the oracle (dropped term, wrong sign, wrong
index, transposed operand, wrong order of the per-token steps) fails at least one of
them; ``test_oracle_mutants.py`` plants such slips to show it.

Each pin takes the loaded oracle library (so a deliberately broken build can be passed
in) and returns a float error; callers compare against ``TOL``.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle

TOL = 1e-10
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example_2x2.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit_rows(rng, *shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_inputs(seed, B=1, T=7, HK=1, HV=1, dk=4, dv=3, h0=True, beta=None, g_zero=False):
    rng = _rng(seed)
    q = rng.standard_normal((B, T, HK, dk)) * dk ** -0.5
    k = _unit_rows(rng, B, T, HK, dk)
    v = rng.standard_normal((B, T, HV, dv))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, HV)))) if beta is None \
        else np.full((B, T, HV), float(beta))
    g = np.zeros((B, T, HV, dk)) if g_zero else -np.log1p(np.exp(rng.standard_normal((B, T, HV, dk))))
    s0 = 0.3 * rng.standard_normal((B, HV, dk, dv)) if h0 else None
    return dict(q=q, k=k, v=v, g=g, beta=b, h0=s0)


def rel(x, ref):
    return oracle.rel_err(x, ref)


# --------------------------------------------------------------------------------------
# hand-worked example (tests/golden/hand_example_2x2.json)
# --------------------------------------------------------------------------------------
def pin_golden(lib, route="sequential", chunk=1):
    with open(GOLDEN) as f:
        gold = json.load(f)
    inp = {k: np.array(v, dtype=np.float64) for k, v in gold["inputs"].items()}
    g = np.log(inp.pop("g_exp"))
    args = dict(q=inp["q"], k=inp["k"], v=inp["v"], g=g, beta=inp["beta"], h0=inp["h0"])
    if route == "sequential":
        o, ht = oracle.sequential(**args, lib=lib)
    else:
        o, ht = oracle.chunked(**args, chunk=chunk, lib=lib)
    exp_o = np.array(gold["expected"]["o"])
    exp_ht = np.array(gold["expected"]["ht"])
    return max(float(np.max(np.abs(o - exp_o))), float(np.max(np.abs(ht - exp_ht))))


# --------------------------------------------------------------------------------------
# P1: beta = 0 leaves only the decay:  S_t = diag(exp(sum_{s<=t} g_s)) h0,  o_t = S_t^T q_t
# --------------------------------------------------------------------------------------
def pin_beta_zero(lib, route="sequential", chunk=4):
    x = random_inputs(11, B=2, T=9, HK=1, HV=2, dk=5, dv=3, beta=0.0)
    o, ht = _run(lib, x, route, chunk)
    G = 2
    err = 0.0
    for b in range(2):
        for h in range(2):
            cum = np.cumsum(x["g"][b, :, h, :], axis=0)            # [T, dk]
            for t in range(9):
                S = np.exp(cum[t])[:, None] * x["h0"][b, h]         # [dk, dv]
                o_ref = S.T @ x["q"][b, t, h // G]
                err = max(err, float(np.max(np.abs(o[b, t, h] - o_ref))))
            S_T = np.exp(cum[-1])[:, None] * x["h0"][b, h]
            err = max(err, float(np.max(np.abs(ht[b, h] - S_T))))
    return err


# --------------------------------------------------------------------------------------
# P2: g = 0, beta = 1, orthonormal keys, h0 = 0  =>  S_T = sum_t k_t v_t^T and
#     S_T^T k_s = v_s for every s (each write lands exactly and later writes are orthogonal)
# --------------------------------------------------------------------------------------
def pin_orthonormal_keys(lib, route="sequential", chunk=3):
    rng = _rng(12)
    dk, dv, T = 6, 4, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T].reshape(1, T, 1, dk)
    x = dict(q=rng.standard_normal((1, T, 1, dk)), k=k, v=rng.standard_normal((1, T, 1, dv)),
             g=np.zeros((1, T, 1, dk)), beta=np.ones((1, T, 1)), h0=None)
    _, ht = _run(lib, x, route, chunk)
    S_ref = sum(np.outer(k[0, t, 0], x["v"][0, t, 0]) for t in range(T))
    err = float(np.max(np.abs(ht[0, 0] - S_ref)))
    for s in range(T):
        err = max(err, float(np.max(np.abs(ht[0, 0].T @ k[0, s, 0] - x["v"][0, s, 0]))))
    return err


# --------------------------------------------------------------------------------------
# P3: beta = 1 and ||k_t|| = 1, any g and h0: right after write t, S_t^T k_t = v_t, so with
#     q_t = k_t the output equals v_t exactly.
# --------------------------------------------------------------------------------------
def pin_exact_write(lib, route="sequential", chunk=4):
    x = random_inputs(13, B=1, T=11, HK=1, HV=2, dk=5, dv=4, beta=1.0)
    x["q"] = x["k"].copy()
    o, _ = _run(lib, x, route, chunk)
    return float(np.max(np.abs(o - x["v"])))


# --------------------------------------------------------------------------------------
# P10: brute force with dense matrices on tiny inputs:
#      S_t = (I - beta_t k_t k_t^T) diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t
# --------------------------------------------------------------------------------------
def brute_force(x):
    q, k, v, g, beta, h0 = (x[n] for n in ("q", "k", "v", "g", "beta", "h0"))
    B, T, HK, dk = q.shape
    HV, dv = v.shape[2], v.shape[3]
    G = HV // HK
    o = np.zeros((B, T, HV, dv))
    ht = np.zeros((B, HV, dk, dv))
    for b in range(B):
        for h in range(HV):
            S = np.zeros((dk, dv)) if h0 is None else h0[b, h].copy()
            for t in range(T):
                kt = k[b, t, h // G]
                M = np.eye(dk) - beta[b, t, h] * np.outer(kt, kt)
                S = M @ np.diag(np.exp(g[b, t, h])) @ S + beta[b, t, h] * np.outer(kt, v[b, t, h])
                o[b, t, h] = S.T @ q[b, t, h // G]
            ht[b, h] = S
    return o, ht


def pin_brute_force(lib, route="sequential", chunk=2, seed=14):
    x = random_inputs(seed, B=2, T=4, HK=1, HV=2, dk=3, dv=4)
    o, ht = _run(lib, x, route, chunk)
    o_ref, ht_ref = brute_force(x)
    return max(rel(o, o_ref), rel(ht, ht_ref))


# --------------------------------------------------------------------------------------
# P9: GQA with HV = G*HK equals running HK' = HV key heads with q, k repeated h -> h // G
# --------------------------------------------------------------------------------------
def pin_gqa_map(lib, route="sequential", chunk=4):
    x = random_inputs(15, B=1, T=6, HK=2, HV=6, dk=4, dv=3)
    o, ht = _run(lib, x, route, chunk)
    G = 3
    idx = np.arange(6) // G
    y = dict(x, q=x["q"][:, :, idx], k=x["k"][:, :, idx])
    o2, ht2 = _run(lib, y, route, chunk)
    return max(rel(o, o2), rel(ht, ht2))


# --------------------------------------------------------------------------------------
# P8: superposition -- outputs are jointly linear in (h0, v) for fixed q, k, g, beta
# --------------------------------------------------------------------------------------
def pin_superposition(lib, route="sequential", chunk=4):
    x = random_inputs(16, B=1, T=10, HK=1, HV=2, dk=4, dv=5)
    o, ht = _run(lib, x, route, chunk)
    xa = dict(x, v=np.zeros_like(x["v"]))
    xb = dict(x, h0=np.zeros_like(x["h0"]))
    oa, hta = _run(lib, xa, route, chunk)
    ob, htb = _run(lib, xb, route, chunk)
    return max(rel(o, oa + ob), rel(ht, hta + htb))


# --------------------------------------------------------------------------------------
# P7: splitting the sequence and carrying ht as the next h0 changes nothing
# --------------------------------------------------------------------------------------
def pin_split_sequence(lib, route="sequential", chunk=4, split=7):
    x = random_inputs(17, B=2, T=13, HK=1, HV=2, dk=4, dv=3)
    o, ht = _run(lib, x, route, chunk)
    first = {n: (a[:, :split] if n != "h0" else a) for n, a in x.items()}
    o1, ht1 = _run(lib, first, route, chunk)
    second = {n: (a[:, split:] if n != "h0" else ht1) for n, a in x.items()}
    o2, ht2 = _run(lib, second, route, chunk)
    return max(rel(np.concatenate([o1, o2], axis=1), o), rel(ht2, ht))


# --------------------------------------------------------------------------------------
# P11: a gate constant across channels gives the chunk intermediates in closed form:
#      A_rs = beta_r exp(gam_r - gam_s) (k_r . k_s) for s < r,  P_rs = exp(gam_r - gam_s) (q_r . k_s)
#      for s <= r, with gam the inclusive prefix of the scalar gate inside the chunk.
#      Always exercises the chunked route (it is the only one with intermediates).
# --------------------------------------------------------------------------------------
def pin_scalar_gate_gram(lib, route="chunked", chunk=8):
    chunk = max(int(chunk), 3)
    x = random_inputs(31, B=1, T=21, HK=1, HV=1, dk=5, dv=4)
    scal = x["g"][..., :1]
    x["g"] = np.repeat(scal, 5, axis=-1)
    _, _, mids = oracle.chunked(**x, chunk=chunk, intermediates=True, lib=lib)
    err = 0.0
    for n in range((21 + chunk - 1) // chunk):
        t0 = n * chunk
        L = min(chunk, 21 - t0)
        gam = np.cumsum(scal[0, t0:t0 + L, 0, 0])
        kk = x["k"][0, t0:t0 + L, 0]
        qq = x["q"][0, t0:t0 + L, 0]
        bb = x["beta"][0, t0:t0 + L, 0]
        dec = np.exp(gam[:, None] - gam[None, :])
        A_ref = np.tril(bb[:, None] * dec * (kk @ kk.T), -1)
        P_ref = np.tril(dec * (qq @ kk.T))
        err = max(err, float(np.max(np.abs(mids["A"][0, 0, n, :L, :L] - A_ref))),
                  float(np.max(np.abs(mids["P"][0, 0, n, :L, :L] - P_ref))))
    return err


def _run(lib, x, route, chunk):
    if route == "sequential":
        return oracle.sequential(**x, lib=lib)
    return oracle.chunked(**x, chunk=chunk, lib=lib)


ALL_PINS = {
    "golden": pin_golden,
    "beta_zero": pin_beta_zero,
    "orthonormal_keys": pin_orthonormal_keys,
    "exact_write": pin_exact_write,
    "brute_force": pin_brute_force,
    "gqa_map": pin_gqa_map,
    "superposition": pin_superposition,
    "split_sequence": pin_split_sequence,
    "scalar_gate_gram": pin_scalar_gate_gram,
}
