"""TEST INFRASTRUCTURE ONLY: fp64 CPU oracle for the channelwise gated delta rule.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The GPU product path (``gated_delta_rule_70_amd``) never imports
it and shares no code with it.

Two routes to the same result, both in fp64 (see ``gdr_oracle.c`` for the arithmetic):

* :func:`sequential` -- the token recurrence (decay, predict, rank-one update, output
  from the updated state), in the order given by the first commit summary of ExecuTorch
  PR #21021 "Reorder channelwise gated delta rule chunked hot loops for
  autovectorization".
* :func:`chunked` -- the chunkwise WY/UT form of the second commit summary of that page,
  with an exact forward-substitution solve; it can export its per-chunk intermediates.
* :func:`tree` -- the same token step over a tree of tokens per batch element (every node
  continues from its parent's state), the setting of the tree-verify solve of uzu PR #576
  ("Support TreeUpdateSolve kernel").
* :func:`l2_normalize_keys`, :func:`neg_softplus` -- the input pre-processing of that page's
  real-scale recipe (normalised keys, softplus decay), which the library can fuse.
* :func:`varlen` -- a packed batch of sequences of different lengths, laid end to end: each
  sequence run through one of the routes above on its own, from its own initial state.
* :func:`gate_per_value_head` -- a gate given per key head, as every value head of the GQA
  group sees it (the per-key-head layout that the uzu PR #576 review thread on the
  per-value-head gram is about).

Inputs may be numpy arrays or torch CPU tensors of any float dtype (bf16 values are
upcast exactly).  Layouts: q, k ``[B,T,HK,dk]``; v ``[B,T,HV,dv]``; g ``[B,T,HV,dk]``, or
``[B,T,HK,dk]`` for a gate shared per key head (expanded by :func:`gate_per_value_head`);
beta ``[B,T,HV]``; h0 ``[B,HV,dk,dv]`` or None.  Results are fp64 numpy arrays.

Parity is pinned by the ``-m "not gpu"`` tests (closed forms, hand-worked example,
brute force with dense matrices, algebraic invariants, planted-mistake checks).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_I64 = ctypes.c_int64
_DP = ctypes.POINTER(ctypes.c_double)


def build(src: str = _SRC, out: str = _LIB_PATH, extra_flags: tuple = ()) -> str:
    """Compile the oracle with gcc (OpenMP over independent (batch, head) pairs)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", *extra_flags,
           "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _needs_build() -> bool:
    return (not os.path.exists(_LIB_PATH)
            or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))


def load(path: str | None = None):
    """Load (building first if missing or stale) and return the ctypes library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if _needs_build():
                build()
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib):
    lib.oracle_gdr_sequential.restype = ctypes.c_int
    lib.oracle_gdr_sequential.argtypes = [_I64] * 6 + [_DP] * 8 + [ctypes.c_int]
    lib.oracle_gdr_chunked.restype = ctypes.c_int
    lib.oracle_gdr_chunked.argtypes = [_I64] * 7 + [_DP] * 14 + [ctypes.c_int]
    lib.oracle_gdr_tree.restype = ctypes.c_int
    lib.oracle_gdr_tree.argtypes = [_I64] * 6 + [_DP] * 6 + [ctypes.POINTER(ctypes.c_int32), _DP,
                                                              ctypes.c_int]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    return lib


def _f64(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: upcast exactly through fp32 -> fp64
        x = x.detach().cpu()
        import torch  # local import: numpy-only callers never need torch

        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_DP)


def gate_per_value_head(g, HV: int) -> np.ndarray:
    """A gate ``[B,T,HK,dk]`` given once per key head -> ``[B,T,HV,dk]``: value head h of a
    GQA group of G = HV / HK contiguous value heads decays with the gate of its key head
    h // G, the same head map as for q and k."""
    g = _f64(g)
    HK = g.shape[2]
    if HV % HK:
        raise ValueError("value heads must be a multiple of key heads")
    return np.repeat(g, HV // HK, axis=2)


def _gate(g, q, v):
    """g as given, or expanded to one row per value head if given per key head."""
    HK, HV = q.shape[2], v.shape[2]
    if g.shape[2] == HK and HK != HV:
        return gate_per_value_head(g, HV)
    return g


def _dims(q, k, v, g, beta, h0):
    B, T, HK, dk = q.shape
    if k.shape != q.shape:
        raise ValueError(f"k shape {k.shape} != q shape {q.shape}")
    Bv, Tv, HV, dv = v.shape
    if (Bv, Tv) != (B, T):
        raise ValueError("v batch/time dims differ from q")
    if g.shape != (B, T, HV, dk):
        raise ValueError(f"g shape {g.shape} != {(B, T, HV, dk)}")
    if beta.shape != (B, T, HV):
        raise ValueError(f"beta shape {beta.shape} != {(B, T, HV)}")
    if h0 is not None and h0.shape != (B, HV, dk, dv):
        raise ValueError(f"h0 shape {h0.shape} != {(B, HV, dk, dv)}")
    if HV % HK:
        raise ValueError("value heads must be a multiple of key heads")
    return B, T, HK, HV, dk, dv


def sequential(q, k, v, g, beta, h0=None, threads: int = 0, lib=None):
    """Token-by-token recurrence in fp64.  Returns ``(o, ht)``."""
    lib = lib or load()
    q, k, v, g, beta, h0 = (_f64(x) for x in (q, k, v, g, beta, h0))
    g = _gate(g, q, v)
    B, T, HK, HV, dk, dv = _dims(q, k, v, g, beta, h0)
    o = np.empty((B, T, HV, dv), np.float64)
    ht = np.empty((B, HV, dk, dv), np.float64)
    rc = lib.oracle_gdr_sequential(B, T, HK, HV, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht), int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_gdr_sequential failed ({rc})")
    return o, ht


def chunked(q, k, v, g, beta, h0=None, chunk: int = 64, threads: int = 0,
            intermediates: bool = False, lib=None):
    """Chunkwise WY/UT form in fp64.  Returns ``(o, ht)`` or ``(o, ht, dict)``.

    The dict (when ``intermediates``) holds per-chunk ``A``, ``P`` ``[B,HV,NC,C,C]``,
    ``W`` and ``gam`` ``[B,HV,NC,C,dk]``, ``Ubar`` and ``U`` ``[B,HV,NC,C,dv]``; rows and
    columns past the end of a ragged last chunk are zero.
    """
    lib = lib or load()
    q, k, v, g, beta, h0 = (_f64(x) for x in (q, k, v, g, beta, h0))
    g = _gate(g, q, v)
    B, T, HK, HV, dk, dv = _dims(q, k, v, g, beta, h0)
    C = int(chunk)
    NC = (T + C - 1) // C
    o = np.empty((B, T, HV, dv), np.float64)
    ht = np.empty((B, HV, dk, dv), np.float64)
    mids = None
    if intermediates:
        mids = {
            "A": np.zeros((B, HV, NC, C, C)),
            "P": np.zeros((B, HV, NC, C, C)),
            "W": np.zeros((B, HV, NC, C, dk)),
            "Ubar": np.zeros((B, HV, NC, C, dv)),
            "U": np.zeros((B, HV, NC, C, dv)),
            "gam": np.zeros((B, HV, NC, C, dk)),
        }
    m = mids or {}
    rc = lib.oracle_gdr_chunked(B, T, HK, HV, dk, dv, C, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht), _ptr(m.get("A")),
                                _ptr(m.get("P")), _ptr(m.get("W")), _ptr(m.get("Ubar")),
                                _ptr(m.get("U")), _ptr(m.get("gam")), int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_gdr_chunked failed ({rc})")
    return (o, ht, mids) if intermediates else (o, ht)


def tree(q, k, v, g, beta, h0, parent, threads: int = 0, lib=None):
    """Token recurrence over a tree, in fp64.  ``parent`` is ``[B,T]`` int with entries in
    ``[-1, t)`` (-1: the node continues from h0, or from zero if h0 is None).  Returns
    ``o`` ``[B,T,HV,dv]``: each node's output from the state at the end of its path."""
    lib = lib or load()
    q, k, v, g, beta, h0 = (_f64(x) for x in (q, k, v, g, beta, h0))
    g = _gate(g, q, v)
    B, T, HK, HV, dk, dv = _dims(q, k, v, g, beta, h0)
    par = np.ascontiguousarray(np.asarray(parent), dtype=np.int32)
    if par.shape != (B, T):
        raise ValueError(f"parent must be [B,T] = {(B, T)}, got {par.shape}")
    o = np.empty((B, T, HV, dv), np.float64)
    rc = lib.oracle_gdr_tree(B, T, HK, HV, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(h0), par.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _ptr(o),
                             int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_gdr_tree failed ({rc})")
    return o


def l2_normalize_keys(k, eps: float = 1e-12) -> np.ndarray:
    """Raw keys [..., dk] -> k / max(|k|_2, eps) over the last axis, in fp64: the key
    normalisation of the real-scale input recipe (uzu PR #576 review: normalised keys),
    which the library's fused prologue (GDR_K_L2NORM) applies per token and key head."""
    k = _f64(k)
    n = np.sqrt(np.sum(k * k, axis=-1, keepdims=True))
    return k / np.maximum(n, eps)


def neg_softplus(a) -> np.ndarray:
    """Gate logits a -> log-decay g = -softplus(a) = -log(1 + e^a), in fp64, in the form
    -(max(a, 0) + log1p(e^-|a|)) that neither overflows nor cancels: the softplus decay of
    the same input recipe, applied by the library's fused prologue (GDR_G_SOFTPLUS)."""
    a = _f64(a)
    return -(np.maximum(a, 0.0) + np.log1p(np.exp(-np.abs(a))))


def varlen(route, q, k, v, g, beta, cu_seqlens, h0=None, **kw):
    """A packed batch: token tensors ``[T, H, d]`` (or ``[1, T, H, d]``), ``cu_seqlens``
    ``[N+1]`` with sequence i on rows ``[cu[i], cu[i+1])``, h0 ``[N,HV,dk,dv]`` or None.  Each
    sequence is passed to ``route`` (:func:`sequential` or :func:`chunked`, extra keywords
    forwarded) as a batch of one with its own h0 row.  Returns ``(o [T,HV,dv], ht
    [N,HV,dk,dv])``; rows outside every sequence stay zero."""
    q, k, v, g, beta, h0 = (_f64(x) for x in (q, k, v, g, beta, h0))
    q, k, v, g, beta = (x[0] if x.ndim == (3 if n == "beta" else 4) else x
                        for n, x in zip(("q", "k", "v", "g", "beta"), (q, k, v, g, beta)))
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    N = len(cu) - 1
    T, HV, dv = v.shape
    dk = q.shape[2]
    if any(b < a for a, b in zip(cu, cu[1:])) or cu[0] < 0 or cu[-1] > T:
        raise ValueError("cu_seqlens must be non-decreasing within [0, T]")
    o = np.zeros((T, HV, dv))
    ht = np.zeros((N, HV, dk, dv))
    for i in range(N):
        a, b = cu[i], cu[i + 1]
        hi = None if h0 is None else h0[i:i + 1]
        if b == a:  # no rows: the state passes through
            ht[i] = 0.0 if hi is None else hi[0]
            continue
        oi, hti = route(q[None, a:b], k[None, a:b], v[None, a:b], g[None, a:b], beta[None, a:b], hi, **kw)
        o[a:b] = oi[0]
        ht[i] = hti[0]
    return o, ht


def num_threads() -> int:
    """Threads an OpenMP region of the oracle uses by default on this host."""
    return int(load().oracle_num_threads())


def rel_err(x, ref) -> float:
    """max|x - ref| / max|ref| over all elements (absolute error if ref is all zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    return num / den if den > 0 else num
