"""Pins for the oracle's tree route (oracle.tree: the token recurrence over a token tree,
every node continuing from its parent's state) and planted mistakes they must catch.

Each pin checks the tree route against something it does not share: the sequential
route (pinned on its own in test_oracle_pins.py) run on a chain or on each node's root
path, single steps from the initial state, and a dense fp64 evaluation of the
ancestry-masked chunk algebra (gram over strict ancestors, causal terms over ancestors and
the node itself, one triangular solve), which is the form the GPU kernel evaluates.
"""
import os

import numpy as np
import pytest

import oracle
from oracle_pins import random_inputs

TOL = 1e-10
SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")


def _tree(kind, B, T, seed):
    rng = np.random.default_rng(seed)
    if kind == "chain":
        return np.tile(np.arange(T, dtype=np.int32) - 1, (B, 1))
    if kind == "star":
        return np.full((B, T), -1, np.int32)
    par = np.empty((B, T), np.int32)
    for b in range(B):
        for t in range(T):
            par[b, t] = rng.integers(-1, t) if t > 0 else -1
    return par


def _path(par_b, r):
    """Node indices from the root down to r."""
    out = []
    while r >= 0:
        out.append(r)
        r = int(par_b[r])
    return out[::-1]


def pin_tree_chain(lib):
    x = random_inputs(31, B=2, T=9, HK=1, HV=2, dk=4, dv=3)
    o_t = oracle.tree(**x, parent=_tree("chain", 2, 9, 0), lib=lib)
    o_s, _ = oracle.sequential(**x)
    return oracle.rel_err(o_t, o_s)


def pin_tree_star(lib):
    x = random_inputs(32, B=2, T=6, HK=1, HV=2, dk=4, dv=3)
    o_t = oracle.tree(**x, parent=_tree("star", 2, 6, 0), lib=lib)
    err = 0.0
    for t in range(6):
        one = {n: (x[n][:, t:t + 1] if n != "h0" else x[n]) for n in x}
        o_s, _ = oracle.sequential(**one)
        err = max(err, oracle.rel_err(o_t[:, t:t + 1], o_s))
    return err


def pin_tree_paths(lib):
    B, T = 2, 12
    x = random_inputs(33, B=B, T=T, HK=2, HV=4, dk=5, dv=3)
    par = _tree("random", B, T, 7)
    o_t = oracle.tree(**x, parent=par, lib=lib)
    err = 0.0
    for b in range(B):
        for r in range(T):
            idx = _path(par[b], r)
            seq = {n: x[n][b:b + 1, idx] for n in ("q", "k", "v", "g", "beta")}
            seq["h0"] = x["h0"][b:b + 1]
            o_s, _ = oracle.sequential(**seq)
            err = max(err, oracle.rel_err(o_t[b, r], o_s[0, -1]))
    return err


def masked_wy(x, par):
    """Dense fp64 evaluation of the ancestry-masked chunk algebra for a whole tree."""
    q, k, v, g, beta, h0 = x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"]
    B, T, HK, dk = q.shape
    HV, dv = v.shape[2], v.shape[3]
    G = HV // HK
    o = np.zeros((B, T, HV, dv))
    for b in range(B):
        anc = [set(_path(par[b], r)[:-1]) for r in range(T)]
        for h in range(HV):
            kh = h // G
            K, Q = k[b, :, kh], q[b, :, kh]
            gam = np.zeros((T, dk))
            for r in range(T):
                gam[r] = g[b, r, h] + (gam[par[b, r]] if par[b, r] >= 0 else 0.0)
            A = np.zeros((T, T))
            P = np.zeros((T, T))
            for r in range(T):
                for s in anc[r] | {r}:
                    e = np.exp(gam[r] - gam[s])
                    P[r, s] = np.sum(Q[r] * K[s] * e)
                    if s != r:
                        A[r, s] = beta[b, r, h] * np.sum(K[r] * K[s] * e)
            S0 = h0[b, h] if h0 is not None else np.zeros((dk, dv))
            Kt, Qt = np.exp(gam) * K, np.exp(gam) * Q
            rhs = beta[b, :, h][:, None] * (v[b, :, h] - Kt @ S0)
            U = np.linalg.solve(np.eye(T) + A, rhs)
            o[b, :, h] = Qt @ S0 + P @ U
    return o


def pin_tree_masked_wy(lib):
    B, T = 2, 10
    x = random_inputs(34, B=B, T=T, HK=1, HV=2, dk=4, dv=3)
    par = _tree("random", B, T, 11)
    return oracle.rel_err(oracle.tree(**x, parent=par, lib=lib), masked_wy(x, par))


TREE_PINS = {"chain": pin_tree_chain, "star": pin_tree_star, "paths": pin_tree_paths,
             "masked_wy": pin_tree_masked_wy}


@pytest.mark.parametrize("name", list(TREE_PINS))
def test_tree_pin(name):
    assert TREE_PINS[name](oracle.load()) < TOL


def test_tree_without_h0_and_gqa():
    x = random_inputs(35, B=1, T=8, HK=2, HV=4, dk=4, dv=2, h0=False)
    par = _tree("random", 1, 8, 5)
    assert oracle.rel_err(oracle.tree(**x, parent=par), masked_wy(x, par)) < TOL


def test_tree_rejects_parent_out_of_range():
    x = random_inputs(36, B=1, T=4, dk=2, dv=2)
    for bad in ([-1, 1, 0, 0], [-2, 0, 0, 0], [-1, 0, 2, 1]):
        with pytest.raises(RuntimeError):
            oracle.tree(**x, parent=np.array([bad], np.int32))


# --------------------------------------------------------------------------------------
# planted mistakes in the tree route (anchors are unique to oracle_gdr_tree)
TREE_MUTANTS = [
    ("tree_continues_previous_node",
     "if (p >= 0)\n                memcpy(S, states + p * dk * dv",
     "if (t > 0)\n                memcpy(S, states + (t - 1) * dk * dv"),
    ("tree_roots_ignore_h0",
     "else if (h0)\n                memcpy(S, h0 + bh * dk * dv",
     "else if (0)\n                memcpy(S, h0 + bh * dk * dv"),
    ("tree_decay_dropped",
     "/* decay */\n            for (int64_t i = 0; i < dk; ++i) {\n                const double e = exp(gt[i]);",
     "/* decay */\n            for (int64_t i = 0; i < dk; ++i) {\n                const double e = 1.0;"),
    ("tree_beta_dropped",
     "d[j] = bt * (vt[j] - pred[j]);\n            for (int64_t i = 0; i < dk; ++i) {\n                const double ki = kt[i];\n                double* Si = S + i * dv;\n                for (int64_t j = 0; j < dv; ++j) Si[j] += ki * d[j];\n            }\n            /* output from the node's updated state */",
     "d[j] = (vt[j] - pred[j]);\n            for (int64_t i = 0; i < dk; ++i) {\n                const double ki = kt[i];\n                double* Si = S + i * dv;\n                for (int64_t j = 0; j < dv; ++j) Si[j] += ki * d[j];\n            }\n            /* output from the node's updated state */"),
    ("tree_output_uses_key",
     "/* output from the node's updated state */\n            for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;\n            for (int64_t i = 0; i < dk; ++i) {\n                const double qi = qt[i];",
     "/* output from the node's updated state */\n            for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;\n            for (int64_t i = 0; i < dk; ++i) {\n                const double qi = kt[i];"),
]


@pytest.mark.parametrize("name,old,new", TREE_MUTANTS, ids=[m[0] for m in TREE_MUTANTS])
def test_tree_pins_catch_planted_mistake(tmp_path, name, old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"anchor of {name} not unique/present"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(str(path), str(tmp_path / "libmutant.so")))
    errors = {}
    for pin_name, pin in TREE_PINS.items():
        try:
            errors[pin_name] = pin(lib)
        except Exception as exc:  # a crash also counts as caught
            errors[pin_name] = float("inf")
    caught = [p for p, e in errors.items() if not (e < TOL)]
    assert caught, f"mutant {name} passed every tree pin: {errors}"
