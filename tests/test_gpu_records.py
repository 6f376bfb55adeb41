"""The chunk-parallel stage on its own: decode the per-chunk records that gdr_chunk_prep
writes to the workspace and compare every operand with the fp64 oracle's chunkwise
intermediates (oracle.chunked(intermediates=True)), so a precision or indexing regression
in one stage shows before the carry mixes it into o and the state.

Record format (the library's workspace layout, per (batch, value head, chunk)): fp16 MFMA
operand fragments of 1 KiB (64 lanes x 8 halves, lane-major).  In a fragment of row tile R
and reduction step K, lane l = 16 g + i and slot j hold the element at row 16 R + i and
reduction index 32 K + 16 (j // 4) + 4 g + j % 4.  In order:
  Qt [nb][kc]  decayed queries (rows: tokens, reduction: key channels), scaled per row
  -W [nb][kc]  negated WY pseudo-keys
  Kb [dkt][nqs] decay-to-end keys, transposed (rows: key channels, reduction: tokens)
  Tb [nb][nqs] (I + A)^-1 diag(beta), lower triangular; steps above a row tile's
               diagonal are not written
  P  [nb][nqs] causal query/key terms, likewise lower triangular, scaled per row
then a 1 KiB fp32 block: exp(gam_last) [dk], Qt row multipliers [C], P row multipliers [C].
Expected values come from the oracle's A, P, W and gam (the solve's inverse by a dense
library solve of the oracle's A); the bar is the parity bar, per operand."""
import numpy as np
import pytest
import torch

import gated_delta_rule_70_amd as gdr
import oracle
from gpu_util import TOL, dev, note, small_inputs

pytestmark = pytest.mark.gpu


def layout(C, dk):
    nb, nqs, kc, dkt = C // 16, (C + 31) // 32, dk // 32, dk // 16
    off = {"qt": 0}
    off["w"] = off["qt"] + nb * kc
    off["kb"] = off["w"] + nb * kc
    off["tb"] = off["kb"] + dkt * nqs
    off["p"] = off["tb"] + nb * nqs
    nfrag = off["p"] + nb * nqs
    return nb, nqs, kc, dkt, off, nfrag, (nfrag + 1) * 1024


def frag_index():
    """(row within tile, reduction index within step) of every (lane, slot)."""
    lane = np.arange(64)[:, None]
    j = np.arange(8)[None, :]
    row = np.broadcast_to(lane % 16, (64, 8))
    red = 16 * (j // 4) + 4 * (lane // 16) + j % 4
    return row, red


def unpack(frags, tiles, steps, rows, cols, written=None):
    """Dense [rows, cols] matrix from fragments [tiles * steps, 64, 8] (fp16)."""
    out = np.zeros((16 * tiles, 32 * steps))
    ri, ki = frag_index()
    for t in range(tiles):
        for k in range(steps):
            if written is not None and not written(t, k):
                continue
            out[16 * t + ri, 32 * k + ki] = frags[t * steps + k]
    return out[:rows, :cols]


def decode(ws, B, T, HV, dk, C):
    nb, nqs, kc, dkt, off, nfrag, nbytes = layout(C, dk)
    NC = -(-T // C)
    raw = ws[: B * HV * NC * nbytes].cpu().numpy().reshape(B * HV, NC, nbytes)
    half = raw[:, :, : nfrag * 1024].copy().view(np.float16).reshape(B * HV, NC, nfrag, 64, 8)
    half = half.astype(np.float64)
    blk = raw[:, :, nfrag * 1024:].copy().view(np.float32).astype(np.float64)
    out = {n: [] for n in ("Qt", "W", "KbT", "Tb", "P", "egl")}
    lower = lambda t, k: 2 * k <= t  # noqa: E731 -- steps of a lower-triangular row tile
    for bh in range(B * HV):
        for n in range(NC):
            f = half[bh, n]
            qsc, psc = blk[bh, n, dk:dk + C], blk[bh, n, dk + C:dk + 2 * C]
            out["Qt"].append(unpack(f[off["qt"]:], nb, kc, C, dk) * qsc[:, None])
            out["W"].append(-unpack(f[off["w"]:], nb, kc, C, dk))
            out["KbT"].append(unpack(f[off["kb"]:], dkt, nqs, dk, C))
            out["Tb"].append(unpack(f[off["tb"]:], nb, nqs, C, C, lower))
            out["P"].append(unpack(f[off["p"]:], nb, nqs, C, C, lower) * psc[:, None])
            out["egl"].append(blk[bh, n, :dk])
    return {k: np.stack(v).reshape(B, HV, NC, *v[0].shape) for k, v in out.items()}


def expected(x, C):
    """The same operands from the oracle's chunkwise intermediates and the inputs."""
    _, _, mids = oracle.chunked(**x, chunk=C, intermediates=True)
    q, k = (x[n].double().numpy() for n in ("q", "k"))
    beta = x["beta"].double().numpy()
    B, T, HK, dk = q.shape
    HV = beta.shape[2]
    G, NC = HV // HK, -(-T // C)
    pad = NC * C - T
    qp = np.pad(q, ((0, 0), (0, pad), (0, 0), (0, 0)))
    kp = np.pad(k, ((0, 0), (0, pad), (0, 0), (0, 0)))
    bp = np.pad(beta, ((0, 0), (0, pad), (0, 0)))
    gam = mids["gam"]  # [B,HV,NC,C,dk], zero past the end of a ragged chunk
    ref = {"W": mids["W"], "P": mids["P"]}
    Qt = np.zeros_like(gam)
    KbT = np.zeros((B, HV, NC, dk, C))
    Tb = np.zeros((B, HV, NC, C, C))
    egl = np.zeros((B, HV, NC, dk))
    for b in range(B):
        for h in range(HV):
            kh = h // G
            for n in range(NC):
                L = min(C, T - n * C)
                rows = slice(n * C, n * C + C)
                g = gam[b, h, n]
                Qt[b, h, n, :L] = np.exp(g[:L]) * qp[b, rows, kh][:L]
                KbT[b, h, n, :, :L] = (np.exp(g[L - 1][None, :] - g[:L]) * kp[b, rows, kh][:L]).T
                inv = np.linalg.solve(np.eye(C) + mids["A"][b, h, n], np.eye(C))
                Tb[b, h, n] = inv * bp[b, rows, h][None, :]
                egl[b, h, n] = np.exp(g[L - 1])
    ref.update(Qt=Qt, KbT=KbT, Tb=Tb, egl=egl)
    return ref


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prep_records_match_oracle_intermediates(C, dtype):
    B, T, HK, HV, dk, dv = 1, 150, 2, 4, 128, 64
    x = small_inputs(B, T, HK, HV, dk, dv, dtype=dtype, seed=C + 3)
    ref = expected(x, C)
    d = dev(x)
    ws = torch.empty(gdr.workspace_bytes(B, T, HK, HV, dk, dv, C), dtype=torch.uint8, device="cuda")
    note(f"prep records C={C} {dtype}")
    gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C, workspace=ws,
                      stage="prep")
    torch.cuda.synchronize()
    got = decode(ws, B, T, HV, dk, C)
    for name in ("Qt", "W", "KbT", "Tb", "P", "egl"):
        e = oracle.rel_err(got[name], ref[name])
        print(f"C={C} {name}: {e:.2e}")
        assert e < TOL, f"{name}: {e:.2e}"


def test_prep_records_scaled_queries():
    """Queries scaled by 2^-20 and 2^12: the stored rows move by exactly that power of two
    into fp16's range and the row multipliers carry it back (decoded values still match)."""
    B, T, HK, HV, dk, dv, C = 1, 100, 2, 4, 128, 64, 64
    for f in (2.0 ** -20, 2.0 ** 12):
        x = small_inputs(B, T, HK, HV, dk, dv, seed=77)
        x["q"] = (x["q"].double() * f).to(torch.bfloat16)
        ref = expected(x, C)
        d = dev(x)
        ws = torch.empty(gdr.workspace_bytes(B, T, HK, HV, dk, dv, C), dtype=torch.uint8, device="cuda")
        note(f"prep records, q * {f}")
        gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C, workspace=ws,
                          stage="prep")
        torch.cuda.synchronize()
        got = decode(ws, B, T, HV, dk, C)
        for name in ("Qt", "P"):
            e = oracle.rel_err(got[name], ref[name])
            assert e < TOL, f"q * {f}: {name} {e:.2e}"
