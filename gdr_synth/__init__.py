"""Seeded synthetic inputs for the channelwise gated delta rule.

This module is shared by the GPU path's tests/benchmark and by the CPU oracle's tests.
It holds only the input recipe (random draws and the elementwise maps that shape them);
none of the method's arithmetic lives here.

Recipe (one ``torch.Generator('cpu')`` per call, seeded; fp32 draws in the fixed order
q, k, v, beta-logits, g-logits, h0):

* ``q = N(0,1) * dk**-0.5``                      (not normalised)
* ``k = n / ||n||_2`` with ``n ~ N(0,1)``        (L2-normalised over dk, in fp32)
* ``v = N(0,1)``
* ``beta = sigmoid(N(0,1))``, or ``U[0.5, 1)`` for the long conditioning-stress case
* ``g = -softplus(N(0,1)) * g_scale``            (per value head and key channel)
* ``h0 = 0.3 * N(0,1)`` in fp32, or ``None``

q/k/v are then rounded to the requested dtype (round-to-nearest-even for bf16); g, beta
and h0 stay fp32.  The magnitudes follow the real-scale recipe requested in the review
of uzu PR #576 (normalised keys, softplus decays, initial state at 0.3 scale).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    HK: int
    HV: int
    dk: int
    dv: int
    chunk: int
    dtype: torch.dtype
    seed: int
    h0: bool
    beta_mode: str = "sigmoid"     # "sigmoid" | "uniform_half"
    g_scale: float = 1.0
    steps: int = 0                 # >0: a decode workload of this many carried steps
    note: str = field(default="", compare=False)


# The shapes of the five workloads the method is measured on.
TINY = Workload("tiny_prefill", B=1, T=64, HK=1, HV=2, dk=32, dv=32, chunk=16,
                dtype=torch.float32, seed=1, h0=False,
                note="tiny prefill, all fp32, GQA 2")
DECODE = Workload("decode_b32", B=32, T=1, HK=16, HV=32, dk=128, dv=128, chunk=64,
                  dtype=torch.bfloat16, seed=2, h0=True, steps=1000,
                  note="decode, 1000 carried steps")
PREFILL_1x4097 = Workload("prefill_b1_t4097", B=1, T=4097, HK=16, HV=32, dk=128, dv=128,
                          chunk=64, dtype=torch.bfloat16, seed=3, h0=False,
                          note="single-sequence prefill, ragged final chunk")
PREFILL_8x512 = Workload("prefill_b8_t512", B=8, T=512, HK=16, HV=32, dk=128, dv=128,
                         chunk=64, dtype=torch.bfloat16, seed=4, h0=True,
                         note="batched prefill with initial state")
PREFILL_8x97 = Workload("prefill_b8_t97", B=8, T=97, HK=16, HV=32, dk=128, dv=128,
                        chunk=64, dtype=torch.bfloat16, seed=41, h0=True,
                        note="batched prefill, ragged last 16-block")
PREFILL_1x32768 = Workload("prefill_b1_t32768", B=1, T=32768, HK=16, HV=32, dk=128,
                           dv=128, chunk=64, dtype=torch.bfloat16, seed=5, h0=True,
                           beta_mode="uniform_half", g_scale=0.1,
                           note="long prefill, slow decay (conditioning stress)")

# Beside the five: two sequences of the single-sequence shape, with initial states.
PREFILL_2x4097 = Workload("prefill_b2_t4097", B=2, T=4097, HK=16, HV=32, dk=128, dv=128,
                          chunk=64, dtype=torch.bfloat16, seed=6, h0=True,
                          note="two sequences of 4097 tokens with initial state")

WORKLOADS = {w.name: w for w in (TINY, DECODE, PREFILL_1x4097, PREFILL_8x512, PREFILL_8x97,
                                 PREFILL_1x32768, PREFILL_2x4097)}


def make_inputs(B: int, T: int, HK: int, HV: int, dk: int, dv: int, *,
                dtype: torch.dtype = torch.bfloat16, seed: int = 0, h0: bool = False,
                beta_mode: str = "sigmoid", g_scale: float = 1.0, gate_heads: str = "value") -> dict:
    """Draw one seeded input set on the CPU.  Returns a dict of CPU tensors.

    ``gate_heads`` "value" draws g ``[B,T,HV,dk]``; "key" draws one gate per key head,
    ``[B,T,HK,dk]``, from the same distribution."""
    if gate_heads not in ("value", "key"):
        raise ValueError(f"unknown gate_heads {gate_heads!r}")
    gen = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn(B, T, HK, dk, generator=gen) * dk ** -0.5
    n = torch.randn(B, T, HK, dk, generator=gen)
    k = n / n.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    v = torch.randn(B, T, HV, dv, generator=gen)
    beta_logits = torch.randn(B, T, HV, generator=gen)
    g_logits = torch.randn(B, T, HV if gate_heads == "value" else HK, dk, generator=gen)
    if beta_mode == "sigmoid":
        beta = torch.sigmoid(beta_logits)
    elif beta_mode == "uniform_half":
        beta = 0.5 + 0.5 * torch.rand(B, T, HV, generator=gen)
    else:
        raise ValueError(f"unknown beta_mode {beta_mode!r}")
    g = -torch.nn.functional.softplus(g_logits) * g_scale
    state = (0.3 * torch.randn(B, HV, dk, dv, generator=gen)) if h0 else None
    return {
        "q": q.to(dtype).contiguous(),
        "k": k.to(dtype).contiguous(),
        "v": v.to(dtype).contiguous(),
        "g": g.float().contiguous(),
        "beta": beta.float().contiguous(),
        "h0": None if state is None else state.float().contiguous(),
    }


TREE_KINDS = ("chain", "star", "random", "binary")


def make_tree(B: int, T: int, kind: str = "random", seed: int = 0) -> torch.Tensor:
    """Parent index of every node of a token tree, one tree per batch element: int32
    ``[B,T]`` with ``parent[b][t]`` in ``[-1, t)`` (nodes in topological order; -1 = a
    child of the initial state).

    chain  -- parent t-1 (a plain sequence)
    star   -- every node a child of the initial state
    random -- parent drawn uniformly from [-1, t)
    binary -- the complete binary tree in breadth-first order: a shallow, wide tree like
              the candidate trees of speculative decoding (depth ~ log2 T)
    """
    if kind == "chain":
        par = torch.arange(T, dtype=torch.int32) - 1
        return par.expand(B, T).contiguous()
    if kind == "star":
        return torch.full((B, T), -1, dtype=torch.int32)
    if kind == "binary":
        t = torch.arange(T, dtype=torch.int32)
        par = torch.where(t == 0, torch.full_like(t, -1), (t - 1) // 2)
        return par.expand(B, T).contiguous()
    if kind == "random":
        gen = torch.Generator("cpu").manual_seed(int(seed))
        u = torch.rand(B, T, generator=gen)
        t = torch.arange(T, dtype=torch.float32)
        return (torch.floor(u * (t + 1)) - 1).to(torch.int32).contiguous()
    raise ValueError(f"unknown tree kind {kind!r}")


def workload_inputs(w: Workload, *, T: int | None = None, B: int | None = None) -> dict:
    """Inputs for a named workload (a decode workload draws all its steps as T=steps)."""
    T = T if T is not None else (w.steps if w.steps else w.T)
    B = B if B is not None else w.B
    return make_inputs(B, T, w.HK, w.HV, w.dk, w.dv, dtype=w.dtype, seed=w.seed, h0=w.h0,
                       beta_mode=w.beta_mode, g_scale=w.g_scale)


def head_group(inputs: dict, b: int, kh: int, G: int) -> dict:
    """Slice one (batch, key-head group): key head ``kh`` and its ``G`` value heads.

    Heads are independent, so the oracle can check sampled groups of a large workload.
    """
    hv = slice(kh * G, (kh + 1) * G)
    out = {
        "q": inputs["q"][b:b + 1, :, kh:kh + 1],
        "k": inputs["k"][b:b + 1, :, kh:kh + 1],
        "v": inputs["v"][b:b + 1, :, hv],
        "g": inputs["g"][b:b + 1, :, hv if inputs["g"].shape[2] == inputs["v"].shape[2] else slice(kh, kh + 1)],
        "beta": inputs["beta"][b:b + 1, :, hv],
        "h0": None if inputs["h0"] is None else inputs["h0"][b:b + 1, hv],
    }
    return {k_: (None if t is None else t.contiguous()) for k_, t in out.items()}
