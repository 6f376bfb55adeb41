#!/usr/bin/env python3
"""Benchmark of the channelwise gated delta rule on one MI355X.

Prints ONE JSON line.  ``value`` is prefill throughput in tokens/s on the single-sequence
prefill workload (B=1, T=4097 with a ragged final chunk, HK=16, HV=32, dk=dv=128,
chunk 64, bf16 q/k/v, fp32 g/beta/state/outputs).  A "step" is one full prefill call
(both kernels: the chunk-parallel stage and the sequential carry).  The same line
carries the decode half of the metric (state GB/s over 1000 carried decode steps at
B=32, HK=16, HV=32, dk=dv=128), the roofline of the dominant kernel, the fp64 CPU
oracle's throughput on the same workload, and the parity error of this run's outputs
against that oracle.  All inputs are seeded synthetic data resident in HBM before timing.

    python bench.py [--steps K] [--warmup W] [--decode-steps N] [--no-cpu-baseline]

The roofline's ``traffic`` (HBM bytes per launch of the dominant kernel) comes from the
committed summary of two rocprofv3 counter runs, used only while the kernel sources still
match the digest recorded with it:

    rocprofv3 --pmc FETCH_SIZE -d <dirF> -o run -f csv -- python3 bench.py --profile-run
    rocprofv3 --pmc WRITE_SIZE -d <dirW> -o run -f csv -- python3 bench.py --profile-run
    python3 bench.py --summarize-pmc <dirF> <dirW>      # -> profiles/hbm_traffic_...md

``--profile-run`` is a short run that also launches one calibration kernel of known
traffic (a 256 MiB fp32 negation: 256 MiB read, 256 MiB written); the counters of every
kernel are scaled by what they read for it.  ``--summarize-stats <dir>`` turns a
``rocprofv3 --kernel-trace --stats`` run into the kernel-time summary under profiles/.

Matrix-core use and the sustained clock come from a third counter run (same rule for the
digest):

    rocprofv3 --kernel-trace --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F16 \
        SQ_INSTS_VALU_MFMA_MOPS_F32 GRBM_GUI_ACTIVE -d <dirU> -o run -f csv \
        -- python3 bench.py --profile-run
    python3 bench.py --summarize-util <dirU>            # -> profiles/mfma_util_...md
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s (HV=32,dk=dv=128) + decode state GB/s, % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak, published
# fp32 vector operations per second without packed fp32 instructions (which the library's
# kernels do not use): 256 CUs x 64 lanes x 2.4 GHz; the published 157.3 TFLOP/s counts
# packed FMAs
VALU_F32_OPS_PEAK = 256 * 64 * 2.4e9

CSRC = os.path.join(ROOT, "gated_delta_rule_70_amd", "csrc")
KERNEL_SOURCES = {  # kernel -> the sources its machine code is built from
    "chunk_prep": ["chunk_prep.hip", "chunk_prep_impl.h", "gdr_device.h", "gdr_launch.h"],
    "chunk_carry": ["chunk_carry.hip", "gdr_device.h", "gdr_launch.h"],
    "carry_full": ["chunk_carry_wide.hip", "gdr_stage.h", "gdr_device.h", "gdr_launch.h"],
    "carry_sum": ["chunk_carry_wide.hip", "gdr_stage.h", "gdr_device.h", "gdr_launch.h"],
    "carry_combine": ["chunk_carry_wide.hip", "gdr_stage.h", "gdr_device.h", "gdr_launch.h"],
    "decode": ["decode.hip", "gdr_device.h", "gdr_launch.h"],
    "fused_recurrent": ["decode.hip", "gdr_device.h", "gdr_launch.h"],
    "tree_verify": ["tree_verify.hip", "gdr_device.h", "gdr_launch.h"],
}
# kernel -> substrings that all appear in its (demangled) name in profiler output; the
# column-split carry is chunk_carry_roles_kernel (one column tile per workgroup) or
# chunk_carry_kernel (several), the whole-head carry's full and summary passes (fp32 o,
# as the benchmark runs them) are carry_wide_kernel<..., false, false> and
# <..., true, false>; the decode step is decode_kernel and a multi-token fused recurrence
# token_kernel
KERNEL_SYMBOL = {"chunk_prep": ("chunk_prep_kernel",), "chunk_carry": ("chunk_carry_",),
                 "carry_full": ("carry_wide_kernel", "false, false>"),
                 "carry_sum": ("carry_wide_kernel", "true, false>"),
                 "carry_combine": ("carry_combine_kernel",),
                 "decode": ("decode_kernel",), "fused_recurrent": ("token_kernel",),
                 "tree_verify": ("tree_verify_kernel",)}
CALIB_BYTES = 256 << 20           # calibration kernel: reads and writes this many bytes
HEADLINE_PROFILE = "prefill_b1_t4097_decode_b32"  # the default run's profile summaries


def _matches(sym, name):
    return all(part in name for part in sym)


def traffic_summary(profile=HEADLINE_PROFILE):
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{profile}.md")


def util_summary(profile=HEADLINE_PROFILE):
    return os.path.join(ROOT, "profiles", f"mfma_util_{profile}.md")
UTIL_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_F32",
                 "GRBM_GUI_ACTIVE"]
SIMD_NUM = 1024                # 256 CUs x 4 SIMDs
XCD_NUM = 8                    # the counter CSV sums GRBM_GUI_ACTIVE over the 8 XCDs


def source_digest(kernel):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _per_dispatch_kib(rows, counter):
    """kernel name -> mean per-dispatch value of `counter` (KiB), summed over the rows of a
    dispatch (one per agent dimension)."""
    disp = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        disp[key] = disp.get(key, 0.0) + float(r["Counter_Value"])
    by_kernel = {}
    for (name, _), v in disp.items():
        by_kernel.setdefault(name, []).append(v)
    return {k: sum(v) / len(v) for k, v in by_kernel.items()}


def summarize_pmc(fetch_dir, write_dir, profile=HEADLINE_PROFILE, run_args="--profile-run"):
    fetch = _per_dispatch_kib(_counter_rows(fetch_dir), "FETCH_SIZE")
    write = _per_dispatch_kib(_counter_rows(write_dir), "WRITE_SIZE")
    calib = [k for k in fetch if "neg" in k.lower()]
    if len(calib) != 1 or calib[0] not in write:
        raise SystemExit(f"calibration kernel not found uniquely: {calib}")
    f_fac = CALIB_BYTES / (fetch[calib[0]] * 1024.0)
    w_fac = CALIB_BYTES / (write[calib[0]] * 1024.0)
    out = {"calibration": {"kernel": calib[0], "bytes_read": CALIB_BYTES, "bytes_written": CALIB_BYTES,
                           "fetch_kib": fetch[calib[0]], "write_kib": write[calib[0]],
                           "fetch_factor": f_fac, "write_factor": w_fac},
           "kernels": {}}
    for kern, sym in KERNEL_SYMBOL.items():
        names = [k for k in fetch if _matches(sym, k)]
        if not names:
            continue
        nm = max(names, key=lambda k: fetch[k])  # the instantiation the workload launches
        fb = fetch[nm] * 1024.0 * f_fac
        wb = write.get(nm, 0.0) * 1024.0 * w_fac
        out["kernels"][kern] = {"symbol": nm, "fetch_kib": fetch[nm], "write_kib": write.get(nm, 0.0),
                                "fetch_bytes": round(fb), "write_bytes": round(wb),
                                "traffic_bytes": round(fb + wb), "source_digest": source_digest(kern)}
    lines = [f"# HBM traffic per launch: {profile}",
             "",
             "Two counter runs of the same short benchmark (FETCH_SIZE, then WRITE_SIZE, KiB per",
             "dispatch), each scaled by what the counter reads for a calibration kernel of known",
             "traffic (a 256 MiB fp32 negation).  `source_digest` identifies the kernel sources the",
             "numbers belong to; bench.py reports them only while the sources still match.",
             "",
             "Commands (repository root, one MI355X):",
             "",
             "```",
             f"rocprofv3 --pmc FETCH_SIZE -d {fetch_dir} -o run -f csv -- python3 bench.py {run_args}",
             f"rocprofv3 --pmc WRITE_SIZE -d {write_dir} -o run -f csv -- python3 bench.py {run_args}",
             f"python3 bench.py --summarize-pmc {fetch_dir} {write_dir} --profile-name {profile}",
             "```",
             "",
             "| kernel | fetch MB | write MB | traffic MB |",
             "|---|---|---|---|"]
    for kern, v in out["kernels"].items():
        lines.append(f"| `{kern}` | {v['fetch_bytes'] / 1e6:.2f} | {v['write_bytes'] / 1e6:.2f} | "
                     f"{v['traffic_bytes'] / 1e6:.2f} |")
    lines += ["", f"Calibration factors: fetch {f_fac:.4f}, write {w_fac:.4f} (bytes per counted byte).",
              "", "```json", json.dumps(out, indent=1), "```", ""]
    with open(traffic_summary(profile), "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {traffic_summary(profile)}")


def _per_dispatch(rows, counter, reduce):
    """kernel name -> list over dispatches of `counter` reduced over the rows of a dispatch
    (one row per agent dimension: SE, SIMD, XCD...)."""
    disp = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        disp.setdefault((r["Kernel_Name"], r["Dispatch_Id"]), []).append(float(r["Counter_Value"]))
    out = {}
    for (name, did), vals in disp.items():
        out.setdefault(name, {})[did] = reduce(vals)
    return out


def _dispatch_ns(d):
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    ns = {}
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                ns[(r["Kernel_Name"], r["Dispatch_Id"])] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return ns


def summarize_util(util_dir, profile=HEADLINE_PROFILE, run_args="--profile-run"):
    """Matrix-core busy fraction (MFMA busy cycles summed over SIMDs / (one XCD's GUI-active
    cycles x SIMDs), the profiler's MfmaUtil) and counted matrix flops (MOPS x 512), per
    launch and per second of traced dispatch time."""
    rows = _counter_rows(util_dir)
    busy = _per_dispatch(rows, "SQ_VALU_MFMA_BUSY_CYCLES", sum)
    m16 = _per_dispatch(rows, "SQ_INSTS_VALU_MFMA_MOPS_F16", sum)
    m32 = _per_dispatch(rows, "SQ_INSTS_VALU_MFMA_MOPS_F32", sum)
    gui = _per_dispatch(rows, "GRBM_GUI_ACTIVE", max)
    dur = _dispatch_ns(util_dir)
    out = {"kernels": {}}
    for kern, sym in KERNEL_SYMBOL.items():
        names = [k for k in gui if _matches(sym, k)]
        if not names:
            continue
        nm = max(names, key=lambda k: max(gui[k].values()))  # the instantiation the workload launches
        ids = sorted(gui[nm])
        ns = [dur[(nm, i)] for i in ids if (nm, i) in dur]
        mean = lambda dct: sum(dct.get(i, 0.0) for i in ids) / len(ids)
        g, b = mean(gui[nm]) / XCD_NUM, mean(busy.get(nm, {}))
        f16, f32 = mean(m16.get(nm, {})) * 512, mean(m32.get(nm, {})) * 512
        t = sum(ns) / len(ns) * 1e-9 if ns else None
        out["kernels"][kern] = {
            "symbol": nm, "dispatches": len(ids), "gui_active_cycles": g, "mfma_busy_cycles": b,
            "mfma_busy_frac": b / (g * SIMD_NUM) if g else None,
            "mfma_f16_flops": f16, "mfma_f32_flops": f32,
            "traced_us": t * 1e6 if t else None,
            "mfma_f16_TFLOPs": f16 / t / 1e12 if t else None,
            "source_digest": source_digest(kern)}
    cmd = ("rocprofv3 --kernel-trace --pmc " + " ".join(UTIL_COUNTERS) +
           f" -d {util_dir} -o run -f csv -- python3 bench.py {run_args}")
    lines = [f"# Matrix-core use and clock per launch: {profile}",
             "",
             "One counter run of the short benchmark with a kernel trace beside it.  MFMA busy =",
             "busy cycles summed over the 1024 SIMDs / (GUI-active cycles of one XCD x 1024), the",
             "profiler's MfmaUtil (the CSV sums GRBM_GUI_ACTIVE over the 8 XCDs); matrix flops =",
             "MOPS x 512 (the counters count add or multiply operations in units of 512).  The",
             "GUI-active window of a dispatch is somewhat longer than its traced time, so the busy",
             "fraction is a slight underestimate and no clock is derived from it; the profiler",
             "serialises dispatches while it counts, so the traced times are not the benchmark's.",
             "`source_digest` identifies the kernel sources; bench.py reports the figures only",
             "while the sources still match.",
             "",
             "Commands (repository root, one MI355X):",
             "",
             "```",
             cmd,
             f"python3 bench.py --summarize-util {util_dir} --profile-name {profile}",
             "```",
             "",
             "| kernel | traced us | MFMA busy | f16 matrix GFLOP | f16 matrix TFLOP/s | f32 matrix GFLOP |",
             "|---|---|---|---|---|---|"]
    for kern, v in out["kernels"].items():
        fmt = lambda x, f: "n/a" if x is None else format(x, f)
        lines.append(f"| `{kern}` | {fmt(v['traced_us'], '.2f')} | {fmt(v['mfma_busy_frac'], '.2%')} | "
                     f"{v['mfma_f16_flops'] / 1e9:.3f} | {fmt(v['mfma_f16_TFLOPs'], '.1f')} | "
                     f"{v['mfma_f32_flops'] / 1e9:.3f} |")
    lines += ["", "```json", json.dumps(out, indent=1), "```", ""]
    with open(util_summary(profile), "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {util_summary(profile)}")


def read_util(kernel, profile=HEADLINE_PROFILE):
    """Matrix-core figures of `kernel` for the current sources, or None."""
    try:
        with open(util_summary(profile)) as f:
            blob = json.loads(f.read().split("```json", 1)[1].split("```", 1)[0])
        k = blob["kernels"][kernel]
    except (OSError, IndexError, KeyError, ValueError):
        return None
    if k.get("source_digest") != source_digest(kernel):
        return None
    return {"mfma_busy_frac": k["mfma_busy_frac"],
            "mfma_f16_flops_counted": k["mfma_f16_flops"], "mfma_f32_flops_counted": k["mfma_f32_flops"]}


def read_traffic(kernel, profile=HEADLINE_PROFILE):
    """Calibrated HBM bytes per launch of `kernel`, or None if there is no summary for the
    current sources."""
    try:
        with open(traffic_summary(profile)) as f:
            text = f.read()
        blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        k = blob["kernels"][kernel]
    except (OSError, IndexError, KeyError, ValueError):
        return None
    if k.get("source_digest") != source_digest(kernel):
        return None
    return k["traffic_bytes"]


def summarize_stats(d, out_name, command):
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# Kernel trace: {out_name}", "", "Command (repository root, one MI355X):", "", "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{100 * float(r['TotalDurationNs']) / tot:.1f}% |")
    path = os.path.join(ROOT, "profiles", out_name.replace(" ", "_") + ".md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {path}")


def prefill_bytes(B, T, HK, HV, dk, dv, elt, h0, g_elt=4, o_elt=4):
    """Algorithmic HBM bytes of one prefill, split by the kernel that must move them.

    prep  : q, k (once per key head), g (g_elt bytes per value), beta
    carry : v, o (o_elt bytes per value), the initial state (if any) and the final state
    """
    prep = B * T * (2 * HK * dk * elt + HV * (dk * g_elt + 4))
    carry = B * T * HV * (dv * elt + dv * o_elt) + B * HV * dk * dv * 4 * (2 if h0 else 1)
    return prep, carry


def prefill_flops(B, T, HV, dk, dv, C):
    """Algorithmic flops of the chunked form, per chunk of L tokens and value head:
    gram + causal terms 2K L^2, solve (K+V) L(L-1), state products 6 L K V, P U V L(L+1).
    Returns (prep, carry) with the gram and the pseudo-key solve in prep."""
    prep = carry = 0
    t = T
    while t > 0:
        L = min(C, t)
        prep += 2 * dk * L * L + dk * L * (L - 1)
        carry += dv * L * (L - 1) + 6 * L * dk * dv + dv * L * (L + 1)
        t -= L
    return prep * B * HV, carry * B * HV


def carry_plan(B, T, HV, dk, dv, C):
    """Which carry the library runs for these dims (its shape rule, restated for reporting):
    the whole-head carry with more than 128 (batch, head) pairs, or, when the heads' 16-column
    tiles fit 256 workgroups, with 256 / heads segments once every segment gets at least 16
    chunks; the column-split carry otherwise."""
    nh, nc = B * HV, -(-T // C)
    if dk != dv or dk not in (64, 128):
        return "column-split"
    if nh > 128:
        return "whole-head, 1 segment"
    if nh * (dv // 16) > 256:
        return "column-split"
    want = 256 // nh
    if nc >= 16 * want:
        return f"whole-head, {want} segments"
    return "column-split"


OTHER_PREFILLS = ("prefill_b8_t512", "prefill_b8_t97", "prefill_b1_t32768", "prefill_b2_t4097")


def bench_io_lean(w, steps=10, warmup=2):
    """The same prefill with g stored as bf16 (GDR_G_BF16), then also with o stored as bf16
    (GDR_O_BF16): per-stage kernel times and throughput, and the path's algorithmic bytes at
    each format."""
    import torch

    elt = 2 if w.dtype == torch.bfloat16 else 4
    out = {}
    for key, o_bf16 in (("bf16 g", False), ("bf16 g and o", True)):
        x, o, ht, wall, prep_ms, carry_ms, _ = bench_prefill(w, steps, warmup, g_bf16=True, o_bf16=o_bf16,
                                                            pre_warm_ms=100.0)
        b_prep, b_carry = prefill_bytes(w.B, w.T, w.HK, w.HV, w.dk, w.dv, elt, w.h0, g_elt=2,
                                        o_elt=2 if o_bf16 else 4)
        kern = prep_ms + carry_ms
        r = {"workload": f"{w.name} with {key}", "prep_ms": round(prep_ms, 5), "carry_ms": round(carry_ms, 5),
             "ms_per_step": round(wall / steps * 1e3, 5), "tokens_per_s": round(w.B * w.T / (wall / steps), 1),
             "path_alg_bytes": b_prep + b_carry,
             "path_hbm_frac": round((b_prep + b_carry) / (kern * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if not o_bf16:
            out = r
        else:
            out["with_bf16_o"] = r
    # where the carry is bound by HBM (the whole-head carry at many heads), o's bytes count most
    from gdr_synth import WORKLOADS
    w8 = WORKLOADS["prefill_b8_t512"]
    x, o, ht, wall, prep_ms, carry_ms, _ = bench_prefill(w8, steps, warmup, o_bf16=True, pre_warm_ms=100.0)
    out["prefill_b8_t512_bf16_o"] = {"prep_ms": round(prep_ms, 5), "carry_ms": round(carry_ms, 5),
                                     "ms_per_step": round(wall / steps * 1e3, 5),
                                     "tokens_per_s": round(w8.B * w8.T / (wall / steps), 1)}
    return out


def bench_prologue(w, steps=10, warmup=2):
    """The fused input prologue (GDR_K_L2NORM | GDR_G_SOFTPLUS) on the headline prefill:
    raw keys and gate logits handed to the library, against the caller doing the key
    normalisation and the softplus decay as separate passes (torch on the GPU) and then
    calling the plain prefill.  Reports both times and the HBM bytes the fusion removes (the
    separate passes read and write k and g once each)."""
    import torch
    import torch.nn.functional as F

    import gated_delta_rule_70_amd as gdr
    from gdr_synth import workload_inputs

    x = workload_inputs(w)
    d = {k: (None if v is None else v.cuda()) for k, v in x.items()}
    gen = torch.Generator("cpu").manual_seed(w.seed + 77)
    a = torch.randn(w.B, w.T, w.HV, w.dk, generator=gen).cuda()   # gate logits
    kraw = (d["k"].float() * 3.0).to(d["k"].dtype)                 # keys off the unit sphere
    B, T, HK, HV, dk, dv, C = w.B, w.T, w.HK, w.HV, w.dk, w.dv, w.chunk
    ws = torch.empty(gdr.workspace_bytes(B, T, HK, HV, dk, dv, C), dtype=torch.uint8, device="cuda")
    o = torch.empty(B, T, HV, dv, device="cuda")
    ht = torch.empty(B, HV, dk, dv, device="cuda")

    def separate():
        kn = F.normalize(kraw.float(), dim=-1).to(kraw.dtype)
        g = -F.softplus(a)
        gdr.chunk_prefill(d["q"], kn, d["v"], g, d["beta"], h0=d["h0"], chunk=C, o=o, ht=ht, workspace=ws)

    def fused():
        gdr.chunk_prefill(d["q"], kraw, d["v"], a, d["beta"], h0=d["h0"], chunk=C, o=o, ht=ht, workspace=ws,
                          k_l2norm=True, g_softplus=True)

    res = {}
    for name, fn in (("separate_passes", separate), ("fused", fused)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) / steps, 5)
    elt = 2 if w.dtype == torch.bfloat16 else 4
    kbytes = B * T * HK * dk * elt
    gbytes = B * T * HV * dk * 4
    return {"workload": f"{w.name}, raw keys and gate logits", "ms_per_step": res,
            "tokens_per_s_fused": round(B * T / (res["fused"] * 1e-3), 1),
            "bytes_removed": 2 * (kbytes + gbytes),
            "what": "the separate passes read and write k (bf16) and g (fp32) once each; "
                    "the fused prologue reads the raw inputs where the kernels already read k and g"}


GATE_HEAD_CASES = ((1, 64), (1, 128), (1, 256), (1, 512), (1, 1024), (1, 2048), (1, 4097), (1, 8192),
                   (1, 16384), (8, 512))


def bench_gate_heads(reps=20, warmup=3):
    """A gate shared per key head (GDR_G_PER_KEY_HEAD) at HK=16 HV=32 dk=dv=128 C=64, bf16
    q/k/v: the chunk-parallel stage in its fused form (a workgroup per value head, the gram
    per value head) and its split form (a workgroup per key head, the gram once per group,
    the solve per value head), timed alone with HIP events over back-to-back calls, for a
    range of sequence lengths -- the crossover the uzu PR #576 review thread asks about --
    and the library's own pick ("auto")."""
    import torch

    import gated_delta_rule_70_amd as gdr
    from gdr_synth import make_inputs

    HK, HV, dk, dv, C = 16, 32, 128, 128, 64
    rows = []
    for B, T in GATE_HEAD_CASES:
        x = make_inputs(B, T, HK, HV, dk, dv, seed=T, gate_heads="key")
        d = {k: (None if v is None else v.cuda()) for k, v in x.items()}
        ws = torch.empty(gdr.workspace_bytes(B, T, HK, HV, dk, dv, C), dtype=torch.uint8, device="cuda")
        o = torch.empty(B, T, HV, dv, device="cuda")
        ht = torch.empty(B, HV, dk, dv, device="cuda")
        row = {"B": B, "T": T}
        for prep in ("fused", "split", "auto"):
            def call():
                gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=C, o=o, ht=ht, workspace=ws,
                                  stage="prep", prep=prep)
            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                call()
            e1.record()
            torch.cuda.synchronize()
            row[f"{prep}_prep_us"] = round(e0.elapsed_time(e1) / reps * 1e3, 2)
        row["faster"] = "split" if row["split_prep_us"] < row["fused_prep_us"] else "fused"
        rows.append(row)
        print(json.dumps(row), flush=True)
        del d, ws, o, ht
    return {"workload": "key-head gate, HK=16 HV=32 dk=dv=128 C=64, bf16 q/k/v", "rows": rows}


def varlen_lengths(n=32, seed=9, lo=1, hi=4097):
    """A seeded mix of sequence lengths, log-uniform on [lo, hi] (many short, a few long)."""
    import numpy as np

    rng = np.random.default_rng(seed)
    return [int(round(float(x))) for x in np.exp(rng.uniform(np.log(lo), np.log(hi), n))]


def bench_long(T=262144, reps=3):
    """One sequence longer than a single launch addresses (HK=16 HV=32 128/128 C=64, bf16,
    h0, the long-prefill recipe): gdr_chunk_prefill runs it as a chain of windows.  Wall time
    per call, CUDA events on the launch stream."""
    import torch

    import gated_delta_rule_70_amd as gdr
    from gdr_synth import make_inputs

    HK, HV, dk, dv, C = 16, 32, 128, 128, 64
    x = make_inputs(1, T, HK, HV, dk, dv, seed=23, h0=True, beta_mode="uniform_half", g_scale=0.1)
    d = {n: (None if t is None else t.cuda()) for n, t in x.items()}
    del x
    print(f"long prefill: inputs of {T} tokens on the device", file=sys.stderr, flush=True)
    need = gdr.workspace_bytes(1, T, HK, HV, dk, dv, C)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.empty(1, T, HV, dv, device="cuda")
    ht = torch.empty(1, HV, dk, dv, device="cuda")

    def call():
        gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C, o=o, ht=ht, workspace=ws)

    call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        call()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    W = 130944  # rows per window at HV=32, 128x128, C=64 (include/gdr.h)
    return {"workload": f"B=1 T={T} HK={HK} HV={HV} {dk}x{dv} C={C} bf16, h0, g_scale 0.1, beta in [0.5, 1)",
            "windows": -(-T // W), "workspace_bytes": need, "ms_per_call": round(ms, 4),
            "tokens_per_s": round(T / (ms * 1e-3), 1), "finite": bool(torch.isfinite(o).all() and torch.isfinite(ht).all())}


def bench_varlen(reps=10, warmup=2):
    """A packed batch of 32 sequences with a log-uniform length mix (1 .. 4097 rows) at
    HK=16 HV=32 128/128 C=64, bf16: one gdr_chunk_prefill_varlen call, against one
    gdr_chunk_prefill per sequence and against one dense call padded to the longest
    sequence (padding rows with beta = 0, whose outputs are discarded).  Wall time per batch,
    CUDA events on the launch stream."""
    import torch

    import gated_delta_rule_70_amd as gdr
    from gdr_synth import make_inputs

    HK, HV, dk, dv, C = 16, 32, 128, 128, 64
    lengths = varlen_lengths()
    N, T = len(lengths), sum(lengths)
    x = make_inputs(1, T, HK, HV, dk, dv, seed=17, h0=False)
    d = {n: t[0].cuda() for n, t in x.items() if t is not None}
    cu_host = [0]
    for L in lengths:
        cu_host.append(cu_host[-1] + L)
    cu = torch.tensor(cu_host, dtype=torch.int32, device="cuda")
    ws = torch.empty(gdr.workspace_bytes_varlen(N, T, HK, HV, dk, dv, C), dtype=torch.uint8, device="cuda")
    o = torch.empty(T, HV, dv, device="cuda")
    ht = torch.empty(N, HV, dk, dv, device="cuda")

    def packed():
        gdr.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, chunk=C, o=o, ht=ht, workspace=ws)

    seqs = []
    for i in range(N):
        a, b = cu_host[i], cu_host[i + 1]
        sl = {n: d[n][a:b].unsqueeze(0) for n in ("q", "k", "v", "g", "beta")}
        wsi = torch.empty(gdr.workspace_bytes(1, b - a, HK, HV, dk, dv, C), dtype=torch.uint8, device="cuda")
        seqs.append((sl, wsi, o[a:b].unsqueeze(0), ht[i:i + 1]))

    def per_sequence():
        for sl, wsi, oi, hi in seqs:
            gdr.chunk_prefill(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], chunk=C, o=oi, ht=hi, workspace=wsi)

    Lmax = max(lengths)
    pad = {n: torch.zeros((N, Lmax) + tuple(d[n].shape[1:]), dtype=d[n].dtype, device="cuda")
           for n in ("q", "k", "v", "g", "beta")}
    for i in range(N):
        for n in pad:
            pad[n][i, :lengths[i]] = d[n][cu_host[i]:cu_host[i + 1]]
    wsp = torch.empty(gdr.workspace_bytes(N, Lmax, HK, HV, dk, dv, C), dtype=torch.uint8, device="cuda")
    op = torch.empty(N, Lmax, HV, dv, device="cuda")

    def padded():
        gdr.chunk_prefill(pad["q"], pad["k"], pad["v"], pad["g"], pad["beta"], chunk=C, o=op, ht=ht, workspace=wsp)

    res = {}
    for name, fn in (("packed", packed), ("per_sequence", per_sequence), ("padded", padded)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) / reps, 4)
    # the padded batch carries its states past each sequence's end (beta = 0 rows still
    # decay), so only its time is comparable, not its final states
    return {"workload": f"{N} sequences, log-uniform lengths 1..4097 ({T} rows, longest {Lmax}), "
                        "HK=16 HV=32 dk=dv=128 C=64, bf16",
            "ms_per_batch": res, "tokens_per_s_packed": round(T / (res["packed"] * 1e-3), 1),
            "lengths": lengths}


OTHER_OUTPUTS = {}  # workload name -> (inputs, o, ht) of the last bench_other_prefills run


def bench_other_prefills(steps=5, warmup=1):
    """The other full-size prefill workloads: per-stage kernel times (HIP events on the launch
    stream, back-to-back calls), throughput, and which carry the library picks (each after
    100 ms of untimed calls, so the few timed steps do not catch the clock ramp)."""
    from gdr_synth import WORKLOADS

    out = []
    for name in OTHER_PREFILLS:
        w = WORKLOADS[name]
        x, o, ht, wall, prep_ms, carry_ms, _ = bench_prefill(w, steps, warmup, pre_warm_ms=100.0)
        out.append({"workload": name, "B": w.B, "T": w.T, "h0": w.h0,
                    "prep_ms": round(prep_ms, 5), "carry_ms": round(carry_ms, 5),
                    "ms_per_step": round(wall / steps * 1e3, 5),
                    "tokens_per_s": round(w.B * w.T / (wall / steps), 1),
                    "carry": carry_plan(w.B, w.T, w.HV, w.dk, w.dv, w.chunk)})
        # this run's outputs, kept on the host for the parity check of the CPU-baseline leg
        OTHER_OUTPUTS[name] = (x, o.cpu(), ht.cpu())
        del o, ht
    return out


def decode_bytes(B, HK, HV, dk, dv, elt):
    return 2 * B * HV * dk * dv * 4 + B * (2 * HK * dk * elt + HV * (dv * elt + dk * 4 + 4 + dv * 4))


def _mean(xs):
    return sum(xs) / len(xs)


def bench_prefill(w, steps, warmup, g_bf16=False, graph=False, pre_warm_ms=0.0, o_bf16=False):
    """Wall time of `steps` back-to-back prefills (gdr_chunk_prefill through the C ABI, its
    arguments marshalled once, so the host enqueues far faster than the GPU runs), then the
    per-stage kernel times from a second pass of the same calls with HIP events on the launch
    stream around each stage (kept out of the timed steps: each event is a marker the stream
    waits on)."""
    import torch

    import gated_delta_rule_70_amd as gdr
    from gdr_synth import workload_inputs

    x = workload_inputs(w)
    d = {k: (None if v is None else v.cuda()) for k, v in x.items()}
    if g_bf16:  # the I/O-lean input format: log-decays stored as bf16
        d["g"] = d["g"].to(torch.bfloat16)
    B, T, HK, HV, dk, dv, C = w.B, w.T, w.HK, w.HV, w.dk, w.dv, w.chunk
    ws = torch.empty(gdr.workspace_bytes(B, T, HK, HV, dk, dv, C), dtype=torch.uint8, device="cuda")
    o = torch.empty(B, T, HV, dv, device="cuda", dtype=torch.bfloat16 if o_bf16 else torch.float32)
    ht = torch.empty(B, HV, dk, dv, device="cuda")
    # one binding call validates the shapes; the timed calls reuse its marshalled arguments
    gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk=C, o=o, ht=ht, workspace=ws)
    L = gdr.lib()
    dims = gdr.Dims(B, T, HK, HV, dk, dv, C, gdr.BF16 if w.dtype == torch.bfloat16 else gdr.F32,
                    (gdr.G_BF16 if g_bf16 else 0) | (gdr.O_BF16 if o_bf16 else 0))
    ptr = lambda t: ctypes.c_void_p(0 if t is None else t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = (ctypes.byref(dims), ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["g"]), ptr(d["beta"]), ptr(d["h0"]),
            ptr(o), ptr(ht), ptr(ws), ctypes.c_size_t(ws.numel()), stream)

    def call(stage):
        fn = {"prep": L.gdr_chunk_prep, "carry": L.gdr_chunk_carry, "both": L.gdr_chunk_prefill}[stage]
        st = fn(*args)
        if st != 0:
            raise RuntimeError(f"{stage}: gdr status {st}")

    # Untimed device warm-up before the warmup steps: the GPU raises its clocks over tens of
    # milliseconds of load, so a few warmup steps alone would time the ramp.
    t_end = time.perf_counter() + pre_warm_ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(10):
            call("both")
        torch.cuda.synchronize()
    for _ in range(warmup):
        call("both")
    torch.cuda.synchronize()
    # the timed steps: plain back-to-back calls, nothing else on the stream
    t0 = time.perf_counter()
    for _ in range(steps):
        call("both")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-kernel times from a second pass over the same calls, events around each stage
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        call("prep")
        e[1].record()
        call("carry")
        e[2].record()
    torch.cuda.synchronize()
    prep_ms = _mean([e[0].elapsed_time(e[1]) for e in ev])
    carry_ms = _mean([e[1].elapsed_time(e[2]) for e in ev])
    graph_ms = None
    if graph:  # `steps` calls captured into one graph and replayed (no host launch cost per call)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for _ in range(steps):
                st = L.gdr_chunk_prefill(*args[:-1], gs)
                if st != 0:
                    raise RuntimeError(f"gdr status {st} under capture")
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        graph_ms = a.elapsed_time(b) / steps
        del g
    return x, o, ht, wall, prep_ms, carry_ms, graph_ms


def bench_decode(w, steps, warmup):
    """Carried decode steps on one state (the workload as defined), then the same number of
    steps cycling over 8 independent states (512 MiB) so the state stream cannot be
    served from the 256 MB last-level cache."""
    import torch

    import gated_delta_rule_70_amd as gdr
    from gdr_synth import make_inputs

    B, HK, HV, dk, dv = w.B, w.HK, w.HV, w.dk, w.dv
    nstep = min(steps, w.steps)
    x = make_inputs(B, nstep, HK, HV, dk, dv, dtype=w.dtype, seed=w.seed, h0=True)
    # per-step contiguous views [B,1,H,d]
    tm = {n: x[n].transpose(0, 1).contiguous().cuda() for n in ("q", "k", "v", "g", "beta")}
    h0 = x["h0"].cuda()
    L = gdr.lib()
    dims = gdr.Dims(B, 1, HK, HV, dk, dv, 0, gdr.BF16)
    obuf = torch.empty(nstep, B, HV, dv, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    args = [(ptr(tm["q"][t]), ptr(tm["k"][t]), ptr(tm["v"][t]), ptr(tm["g"][t]), ptr(tm["beta"][t]),
             ptr(obuf[t])) for t in range(nstep)]

    def run(states, timed):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(nstep)] if timed else None
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(nstep):
            s = ptr(states[t % len(states)])
            q, k, v, g, b, o = args[t]
            if timed:
                ev[t][0].record()
            st = L.gdr_decode_step(ctypes.byref(dims), q, k, v, g, b, s, o, s, stream)
            if st != 0:
                raise RuntimeError(f"gdr_decode_step failed: {st}")
            if timed:
                ev[t][1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = [a.elapsed_time(b) for a, b in ev] if timed else []
        return wall, per

    scratch = [h0.clone()]
    for _ in range(max(1, warmup)):
        run(scratch, False)
    state = h0.clone()
    wall_c, per_c = run([state], True)
    rot = [h0.clone() for _ in range(8)]
    wall_r, per_r = run(rot, True)
    per_c.sort()
    per_r.sort()

    # The same carried steps replayed from one captured graph (no host launch cost).
    gstate = h0.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        s = ptr(gstate)
        for t in range(nstep):
            q, k, v, g, b, o = args[t]
            st = L.gdr_decode_step(ctypes.byref(dims), q, k, v, g, b, s, o, s, cs)
            if st != 0:
                raise RuntimeError(f"gdr_decode_step failed under capture: {st}")
    graph.replay()
    torch.cuda.synchronize()
    ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ga.record()
    graph.replay()
    gb.record()
    torch.cuda.synchronize()
    graph_ms = ga.elapsed_time(gb) / nstep
    del graph

    # The same steps cycling over the 8 states (512 MiB, more than the 256 MB last-level
    # cache), replayed from a graph: the HBM-resident decode rate without host launch gaps.
    rgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(rgraph):
        cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for t in range(nstep):
            q, k, v, g, b, o = args[t]
            s = ptr(rot[t % len(rot)])
            st = L.gdr_decode_step(ctypes.byref(dims), q, k, v, g, b, s, o, s, cs)
            if st != 0:
                raise RuntimeError(f"gdr_decode_step failed under capture: {st}")
    rgraph.replay()
    torch.cuda.synchronize()
    ga.record()
    rgraph.replay()
    gb.record()
    torch.cuda.synchronize()
    graph_rot_ms = ga.elapsed_time(gb) / nstep
    del rgraph

    # Attainable HBM rate: one 1 GiB device copy (1 GiB read + 1 GiB written), far larger
    # than the last-level cache.
    big = 1 << 28
    bsrc = torch.ones(big, device="cuda")
    bdst = torch.empty_like(bsrc)
    bdst.copy_(bsrc)
    torch.cuda.synchronize()
    ga.record()
    for _ in range(5):
        bdst.copy_(bsrc)
    gb.record()
    torch.cuda.synchronize()
    copy_1g_ms = ga.elapsed_time(gb) / 5
    del bsrc, bdst

    # A plain device copy of the state's size (read + write the same bytes as one step's
    # state stream), cycling over 8 buffer pairs like the rotating decode run.
    nel = B * HV * dk * dv
    srcs = [torch.randn(nel, device="cuda") for _ in range(8)]
    dsts = [torch.empty(nel, device="cuda") for _ in range(8)]
    for i in range(8):
        dsts[i].copy_(srcs[i])
    torch.cuda.synchronize()
    ca, cb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 80
    ca.record()
    for i in range(reps):
        dsts[i % 8].copy_(srcs[i % 8])
    cb.record()
    torch.cuda.synchronize()
    copy_ms = ca.elapsed_time(cb) / reps
    del srcs, dsts
    return {
        "nstep": nstep,
        "carried": {"wall_s": wall_c, "mean_ms": _mean(per_c), "median_ms": per_c[len(per_c) // 2]},
        "rotating8": {"wall_s": wall_r, "mean_ms": _mean(per_r), "median_ms": per_r[len(per_r) // 2]},
        "graph_ms_per_step": graph_ms, "graph_rot_ms_per_step": graph_rot_ms, "copy_ms": copy_ms,
        "copy_1g_ms": copy_1g_ms,
        "inputs": x, "obuf": obuf, "state": state,
    }


SHORT_T = (1, 2, 4, 8, 16, 32, 64)


def bench_short_calls(w, reps=10):
    """Short multi-token calls at the decode workload's shape: for each T, one call's time
    as T decode launches, as one fused-recurrent launch and as the chunked prefill (best of
    chunk 16/32/64), all on the same inputs, calls issued back to back and timed with HIP
    events on the launch stream."""
    import torch

    import gated_delta_rule_70_amd as gdr
    from gdr_synth import make_inputs

    B, HK, HV, dk, dv = w.B, w.HK, w.HV, w.dk, w.dv
    tmax = max(SHORT_T)
    x = make_inputs(B, tmax, HK, HV, dk, dv, dtype=w.dtype, seed=w.seed + 7, h0=True)
    d = {k: v.cuda() for k, v in x.items()}
    state = d["h0"].clone()
    out = {"T": list(SHORT_T), "decode_loop_ms": [], "fused_recurrent_ms": [], "chunked_ms": [],
           "chunked_best_chunk": [], "fused_recurrent_state_GBps": [], "fused_recurrent_valu_frac": [],
           "fastest": []}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    for T in SHORT_T:
        sl = {n: d[n][:, :T].contiguous() for n in ("q", "k", "v", "g", "beta")}
        steps = [{n: d[n][:, t:t + 1].contiguous() for n in ("q", "k", "v", "g", "beta")} for t in range(T)]
        o = torch.empty(B, T, HV, dv, device="cuda")
        o1 = torch.empty(B, 1, HV, dv, device="cuda")

        def loop():
            for st in steps:
                gdr.decode_step(st["q"], st["k"], st["v"], st["g"], st["beta"], state, o=o1)

        def fused():
            gdr.fused_recurrent(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], h0=state, o=o, ht=state)

        t_loop, t_fused = timed(loop), timed(fused)
        best = None
        for C in (16, 32, 64):
            if C > 16 and C > T:
                continue
            ws = torch.empty(gdr.workspace_bytes(B, T, HK, HV, dk, dv, C), dtype=torch.uint8, device="cuda")

            def chunked():
                gdr.chunk_prefill(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], h0=state, chunk=C, o=o,
                                  ht=state, workspace=ws)

            tc = timed(chunked)
            if best is None or tc < best[0]:
                best = (tc, C)
            del ws
        out["decode_loop_ms"].append(round(t_loop, 5))
        out["fused_recurrent_ms"].append(round(t_fused, 5))
        out["chunked_ms"].append(round(best[0], 5))
        out["chunked_best_chunk"].append(best[1])
        out["fused_recurrent_state_GBps"].append(round(2 * B * HV * dk * dv * 4 / (t_fused * 1e-3) / 1e9, 1))
        # 4 vector operations per state element per token: decay, prediction, update, output
        out["fused_recurrent_valu_frac"].append(
            round(4 * B * HV * dk * dv * T / (t_fused * 1e-3) / VALU_F32_OPS_PEAK, 4))
        out["fastest"].append(min((t_loop, "decode_loop"), (t_fused, "fused_recurrent"),
                                  (best[0], "chunked"))[1])
    out["workload"] = (f"B={B} HK={HK} HV={HV} dk=dv={dk} bf16 q/k/v, h0 given, one call of T tokens; "
                       f"{reps} calls back to back per figure")
    out["valu_peak_ops_per_s"] = VALU_F32_OPS_PEAK
    return out


TREE_CASES = ((1, 33, "binary"), (1, 49, "binary"), (1, 64, "binary"), (1, 64, "random"),
              (1, 64, "chain"), (8, 64, "binary"))


def bench_tree(w, reps=20):
    """Tree-verify solve at the decode workload's head shape (HK=16, HV=32, dk=dv=128, h0
    given) on the tree sizes of the uzu tree-solve measurements: one call's time, calls
    issued back to back and timed with HIP events."""
    import torch

    import gated_delta_rule_70_amd as gdr
    from gdr_synth import make_inputs, make_tree

    out = []
    for B, T, kind in TREE_CASES:
        x = make_inputs(B, T, w.HK, w.HV, w.dk, w.dv, dtype=w.dtype, seed=w.seed + 11, h0=True)
        d = {k: v.cuda() for k, v in x.items()}
        par = make_tree(B, T, kind, seed=w.seed).cuda()
        o = torch.empty(B, T, w.HV, w.dv, device="cuda")

        def call():
            gdr.tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], par, h0=d["h0"], o=o)

        call()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            call()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        # algorithmic work: inputs and outputs once; per head the ancestry-masked gram and
        # causal terms (2 dk flops per ancestor pair), keys/queries times h0 (4 T dk dv),
        # the substitution (2 dv per ancestor pair) and P U (2 dv per pair incl. the node)
        p = par.cpu()
        pairs = 0
        for bb in range(B):
            for t in range(T):
                r = int(p[bb, t])
                while r >= 0:
                    pairs += 1
                    r = int(p[bb, r])
        pairs_h = pairs * w.HV
        flops = (pairs_h * 2 * w.dk * 2 + B * T * w.HV * w.dk * 2 * w.dk  # A and P (incl. diagonal)
                 + 4 * B * T * w.HV * w.dk * w.dv                           # Kt h0, Qt h0
                 + pairs_h * 2 * w.dv + (pairs_h + B * T * w.HV) * 2 * w.dv)
        elt = 2 if w.dtype == torch.bfloat16 else 4
        nbytes = (B * T * (2 * w.HK * w.dk * elt + w.HV * (w.dv * elt + w.dk * 4 + 4 + w.dv * 4))
                  + B * w.HV * w.dk * w.dv * 4 + B * T * 4)
        out.append({"B": B, "T": T, "tree": kind, "us_per_call": round(ms * 1e3, 2),
                    "nodes_per_s": round(B * T / (ms * 1e-3), 1), "alg_flops": flops,
                    "alg_bytes": nbytes, "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                    "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 3)})
    return {"workload": f"HK={w.HK} HV={w.HV} dk=dv={w.dk} bf16 q/k/v, h0 given; {reps} calls back to back",
            "cases": out}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--pre-warm-ms", type=float, default=300.0,
                    help="untimed device warm-up (repeated prefills) before the warmup steps, so the "
                         "timed steps do not measure the clock ramp; reported in the JSON line")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-short-calls", action="store_true")
    ap.add_argument("--workload", default="prefill_b1_t4097")
    ap.add_argument("--profile-run", action="store_true",
                    help="short run for counter collection, plus the calibration kernel")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-util", metavar="UTIL_DIR")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("DIR", "NAME", "COMMAND"))
    ap.add_argument("--section", choices=("tree", "short_calls", "prologue", "gate_heads", "varlen", "long"),
                    help="run only this part of the benchmark (tree-verify cases or short calls) "
                         "and print its JSON; for kernel traces of those kernels")
    ap.add_argument("--profile-name", default=HEADLINE_PROFILE,
                    help="profile summaries to write: the default run's, or a prefill workload's "
                         "(counter runs of `--profile-run --workload <name> --no-decode`)")
    args = ap.parse_args()
    run_args = ("--profile-run" if args.profile_name == HEADLINE_PROFILE
                else f"--profile-run --workload {args.profile_name} --no-decode")
    if args.summarize_util:
        summarize_util(args.summarize_util, args.profile_name, run_args)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, profile=args.profile_name, run_args=run_args)
        return
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.profile_run:
        args.steps, args.warmup, args.decode_steps, args.no_cpu_baseline = 3, 1, 50, True
        args.pre_warm_ms = 0.0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the recurrence's (batch, head) pairs are independent, "
              "so a multi-GPU run is N independent copies of this one; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_70_amd as gdr  # noqa: F401  (fails loudly if libgdr.so is missing)
    from gdr_synth import DECODE, WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.section:
        if args.section == "prologue":
            from gdr_synth import WORKLOADS
            res = bench_prologue(WORKLOADS[args.workload])
        elif args.section == "gate_heads":
            res = bench_gate_heads()
        elif args.section == "varlen":
            res = bench_varlen()
        elif args.section == "long":
            res = bench_long()
        else:
            res = bench_tree(DECODE) if args.section == "tree" else bench_short_calls(DECODE)
        print(json.dumps({"section": args.section, **res}), flush=True)
        return
    w = WORKLOADS[args.workload]
    elt = 2 if w.dtype == torch.bfloat16 else 4
    if args.profile_run:  # calibration kernel of known traffic for the counter runs
        xc = torch.ones(CALIB_BYTES // 4, device="cuda")
        yc = torch.empty_like(xc)
        torch.neg(xc, out=yc)
        torch.cuda.synchronize()
        del xc, yc
    x, o, ht, wall, prep_ms, carry_ms, graph_ms = bench_prefill(w, args.steps, args.warmup,
                                                                 graph=not args.profile_run,
                                                                 pre_warm_ms=args.pre_warm_ms)
    ntok = w.B * w.T
    ms_per_step = wall / args.steps * 1e3
    value = ntok / (wall / args.steps)
    b_prep, b_carry = prefill_bytes(w.B, w.T, w.HK, w.HV, w.dk, w.dv, elt, w.h0)
    f_prep, f_carry = prefill_flops(w.B, w.T, w.HV, w.dk, w.dv, w.chunk)
    kern_ms = prep_ms + carry_ms
    dom = "chunk_carry" if carry_ms >= prep_ms else "chunk_prep"
    dom_ms = max(prep_ms, carry_ms)
    dom_bytes = b_carry if dom == "chunk_carry" else b_prep
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic(dom),
                "alg_bytes_per_launch": dom_bytes, "avg_launch_ms": round(dom_ms, 5)}
    path_gbs = (b_prep + b_carry) / (kern_ms * 1e-3) / 1e9
    path_tflops = (f_prep + f_carry) / (kern_ms * 1e-3) / 1e12
    # the path's ceiling: its algorithmic bytes at HBM peak or its flops at MFMA peak
    ceil_ms = max((b_prep + b_carry) / (HBM_PEAK_GBS * 1e9), (f_prep + f_carry) / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
    # both stages against the HBM peak by their own algorithmic bytes (the roofline line above
    # is the longer one's)
    per_kernel = {}
    for k, ms, nb in (("chunk_prep", prep_ms, b_prep), ("chunk_carry", carry_ms, b_carry)):
        gbs = nb / (ms * 1e-3) / 1e9
        per_kernel[k] = {"achieved": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "alg_bytes_per_launch": nb, "traffic": read_traffic(k)}
    prefill = {
        "kernels_ms": {"chunk_prep": round(prep_ms, 5), "chunk_carry": round(carry_ms, 5)},
        "kernels_hbm": per_kernel,
        "path_alg_bytes": b_prep + b_carry, "path_alg_flops": f_prep + f_carry,
        "path_hbm_GBps": round(path_gbs, 1), "path_hbm_frac": round(path_gbs / HBM_PEAK_GBS, 4),
        "path_mfma_TFLOPs": round(path_tflops, 2),
        "path_frac_of_bf16_mfma_peak": round(path_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "ceiling_ms": round(ceil_ms, 5), "path_frac_of_ceiling": round(ceil_ms / kern_ms, 4),
        "tokens_per_s_kernel_time": round(ntok / (kern_ms * 1e-3), 1),
        "carry": carry_plan(w.B, w.T, w.HV, w.dk, w.dv, w.chunk),
        # the timed steps captured into one HIP graph and replayed: no host launch cost
        "graph_replay": None if graph_ms is None else {
            "ms_per_step": round(graph_ms, 5), "tokens_per_s": round(ntok / (graph_ms * 1e-3), 1)},
        "counters": {"chunk_prep": read_util("chunk_prep"), "chunk_carry": read_util("chunk_carry")},
    }

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "pre_warm_ms": args.pre_warm_ms,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "arithmetic": "fp16 MFMA operands with fp32 accumulation; fp32 state, decay "
                                       "factors, diagonal gram tiles and triangular solve",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} T={w.T} HK={w.HK} HV={w.HV} dk={w.dk} dv={w.dv} "
                               f"chunk={w.chunk} bf16 q/k/v, fp32 g/beta/state/o, h0={'yes' if w.h0 else 'no'}",
                   "global_batch": w.B, "seq_len": w.T, "parallelism": "single GPU"},
        "roofline": roofline, "prefill": prefill,
    }

    if not args.no_decode:
        dres = bench_decode(DECODE, args.decode_steps, 10)
        dbytes = decode_bytes(DECODE.B, DECODE.HK, DECODE.HV, DECODE.dk, DECODE.dv, 2)
        sbytes = 2 * DECODE.B * DECODE.HV * DECODE.dk * DECODE.dv * 4
        dec = {"workload": f"decode_b32: B={DECODE.B} HK={DECODE.HK} HV={DECODE.HV} dk=dv={DECODE.dk} "
                           f"bf16 q/k/v, {dres['nstep']} carried steps",
               "alg_bytes_per_step": dbytes, "state_bytes_per_step": sbytes}
        for mode in ("carried", "rotating8"):
            r = dres[mode]
            gbs = dbytes / (r["mean_ms"] * 1e-3) / 1e9
            dec[mode] = {"avg_launch_ms": round(r["mean_ms"], 5), "median_launch_ms": round(r["median_ms"], 5),
                         "wall_ms_per_step": round(r["wall_s"] / dres["nstep"] * 1e3, 5),
                         "state_GBps": round(sbytes / (r["mean_ms"] * 1e-3) / 1e9, 1),
                         "total_GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        gms = dres["graph_ms_per_step"]
        dec["graph_replay"] = {"ms_per_step": round(gms, 5), "total_GBps": round(dbytes / (gms * 1e-3) / 1e9, 1),
                               "hbm_frac": round(dbytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        grms = dres["graph_rot_ms_per_step"]
        dec["graph_replay_rotating8"] = {
            "what": "the steps cycling over 8 states (512 MiB, HBM-resident), replayed from one graph",
            "ms_per_step": round(grms, 5), "total_GBps": round(dbytes / (grms * 1e-3) / 1e9, 1),
            "hbm_frac": round(dbytes / (grms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        cms = dres["copy_ms"]
        dec["copy_reference"] = {"what": f"device copy of {sbytes // 2} B (state-sized read + write), 8 rotating buffers",
                                 "ms": round(cms, 5), "GBps": round(sbytes / (cms * 1e-3) / 1e9, 1),
                                 "decode_rotating8_frac_of_copy": round(cms / dres["rotating8"]["mean_ms"], 4)}
        c1 = dres["copy_1g_ms"]
        copy_gbs = 2 * (1 << 30) / (c1 * 1e-3) / 1e9
        dec["copy_1GiB"] = {"what": "one 1 GiB device copy (read + write 2 GiB): the attainable HBM rate",
                            "ms": round(c1, 4), "GBps": round(copy_gbs, 1), "hbm_frac": round(copy_gbs / HBM_PEAK_GBS, 4),
                            "decode_graph_rotating8_frac_of_copy":
                                round(dbytes / (grms * 1e-3) / 1e9 / copy_gbs, 4)}
        line["decode"] = dec

    if not args.no_short_calls and not args.profile_run:
        line["short_calls"] = bench_short_calls(DECODE)
        line["tree_verify"] = bench_tree(DECODE)
        line["other_prefills"] = bench_other_prefills()
        line["io_lean"] = bench_io_lean(w)
        line["prologue"] = bench_prologue(w)

    if not args.no_cpu_baseline:
        import numpy as np

        import oracle

        # the full workload, repeated until about 10 s of CPU time have been spent (<= 30 runs)
        runs, t0 = 0, time.perf_counter()
        while True:
            o_ref, ht_ref = oracle.sequential(**x)
            runs += 1
            cpu_s = time.perf_counter() - t0
            if cpu_s >= 10.0 or runs >= 30:
                break
        line["cpu_baseline"] = {"value": round(runs * ntok / cpu_s, 1), "unit": "tokens/s",
                                "cores": oracle.num_threads(), "kind": "oracle",
                                "sample": f"the full {w.name} workload ({ntok} tokens x {w.HV} value heads), "
                                          f"fp64 sequential recurrence, {runs} runs in {cpu_s:.1f} s"}
        # the same recurrence on one host thread, over one key head's group of value heads
        # (a bounded sample), scaled to the whole workload's tokens per second
        from gdr_synth import head_group

        G = w.HV // w.HK
        sub = head_group(x, 0, 0, G)
        t1 = time.perf_counter()
        oracle.sequential(**sub, threads=1)
        one_s = time.perf_counter() - t1
        line["cpu_baseline"]["single_thread"] = {
            "value": round(ntok / (one_s * w.B * w.HK), 1), "unit": "tokens/s", "cores": 1,
            "sample": f"one key head's {G} value heads of {w.name} (batch 0), {one_s:.2f} s, "
                      f"scaled by the {w.B * w.HK} such groups of the workload"}
        line["parity_vs_oracle"] = {
            "o": float(oracle.rel_err(o.double().cpu().numpy(), o_ref)),
            "state": float(oracle.rel_err(ht.double().cpu().numpy(), ht_ref)),
            "tolerance": 2e-3}
        # the other full-size prefills of this run, every head, against the same oracle
        # (for the long conditioning-stress sequence this is its final-state error)
        for name, (xo, oo, hto) in OTHER_OUTPUTS.items():
            oref, htref = oracle.sequential(**xo)
            line["parity_vs_oracle"][name] = {
                "o": float(oracle.rel_err(oo.double().numpy(), oref)),
                "state": float(oracle.rel_err(hto.double().numpy(), htref))}
            del oref, htref
        del np
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
