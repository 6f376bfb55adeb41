"""Helpers for the GPU parity tests (HIP path vs the fp64 oracle)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from gdr_synth import head_group, make_inputs

# Parity bar: max|x - x_ref| / max|x_ref| over all elements, separately for the outputs o
# and for the final state, against the fp64 oracle (bf16 q/k/v and fp32 state).
TOL = 2e-3


def note(msg: str):
    """Name the case before a GPU step, flushed, so a failing run still says what ran."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev(inputs: dict) -> dict:
    return {k: (None if v is None else v.cuda()) for k, v in inputs.items()}


def err(x, ref) -> float:
    if isinstance(x, torch.Tensor):
        x = x.detach().double().cpu().numpy()
    return oracle.rel_err(x, ref)


def small_inputs(B, T, HK, HV, dk, dv, dtype=torch.bfloat16, seed=0, h0=True, **kw):
    return make_inputs(B, T, HK, HV, dk, dv, dtype=dtype, seed=seed, h0=h0, **kw)


def sampled_groups(B: int, HK: int, n: int, seed: int):
    """n distinct (batch, key head) groups, always including the first and the last."""
    rng = np.random.default_rng(seed)
    all_g = [(b, kh) for b in range(B) for kh in range(HK)]
    pick = {all_g[0], all_g[-1]}
    while len(pick) < min(n, len(all_g)):
        pick.add(all_g[int(rng.integers(len(all_g)))])
    return sorted(pick)


def oracle_on_groups(inputs: dict, groups, G: int, threads: int = 0):
    """fp64 oracle outputs for each sampled group: {(b, kh): (o [T,G,dv], ht [G,dk,dv])}."""
    out = {}
    for (b, kh) in groups:
        sub = head_group(inputs, b, kh, G)
        o, ht = oracle.sequential(**sub, threads=threads)
        out[(b, kh)] = (o[0], ht[0])
    return out


def bf16_exact_unit_keys(B, T, HK, dk, seed):
    """Unit-norm keys whose entries are exact in bf16 and fp16: dk/2 entries of
    +-sqrt(2/dk) (a power of two for dk = 32, 128), the rest zero."""
    assert dk in (32, 128)
    val = (2.0 / dk) ** 0.5
    gen = torch.Generator("cpu").manual_seed(seed)
    k = torch.zeros(B, T, HK, dk)
    for idx in np.ndindex(B, T, HK):
        perm = torch.randperm(dk, generator=gen)[: dk // 2]
        sign = torch.randint(0, 2, (dk // 2,), generator=gen) * 2 - 1
        k[idx][perm] = sign.float() * val
    return k


def token_err(x, ref) -> float:
    """Largest per-token relative error: for every token t (axis 1 of [B,T,HV,dv]),
    max|x_t - ref_t| / max|ref_t| over the batch, heads and values, then the maximum over t.
    Unlike the whole-tensor bar it constrains late tokens of a decaying sequence, whose
    outputs are many orders of magnitude below the first ones."""
    if isinstance(x, torch.Tensor):
        x = x.detach().double().cpu().numpy()
    num = np.abs(x - ref).max(axis=(0, 2, 3))
    den = np.abs(ref).max(axis=(0, 2, 3))
    if (den == 0).any():
        raise ValueError("a token has an all-zero reference output")
    return float((num / den).max())
