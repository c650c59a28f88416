#!/usr/bin/env python3
"""Attention-backward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5] [--no-extra] [--no-cpu-baseline]

A step is one complete C-ABI call (row statistics, schedule upload, index, every kernel)
over one batch of synthetic input already resident in HBM.  The headline workload is
the largest single-GPU one, selected bf16 at S = 128K (N1 64, N2 4, D 192 / 128, blocks
of 64, 32 per token); `extra` holds one line each for the dense varlen bf16 workload
(causal, rope 128 + 64, GQA 32/8, four seeded lengths), selected at S = 32K, the
Zipf-skewed varlen selected workload in both determinism settings, the selected backward
at S = 32K without attentionOut, the selected forward at S = 128K and S = 32K, and the
lightning-indexer backward (one 8K sequence, 64 heads, topK 2048) with either dK mode.
`value` is algorithmic TFLOP/s: attended (query row, key row) pairs x 2(3 D_qk + 2 D_v),
causal pairs only (the five GEMMs S, dP, dV, dQ, dK; recomputation is not counted).
Before the warmup calls every workload repeats its call for --prewarm-ms of GPU time, so
that the timed calls run at the sustained clock.

O and the softmax statistics fed to the timed call are produced once, before timing:
for the selected workloads by the library's own forward (attn_fwd_selected, which
the extra lines also time on its own), for the dense one by a plain fp32 torch
forward on the GPU.  The float64 oracle runs only in the CPU-baseline leg, on a
bounded sample of the same workload.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import sparse_attention_backward_amd as sab  # noqa: E402
import workloads as W  # noqa: E402

METRIC = "selected/dense attention-backward TFLOP/s and % of bf16 MFMA peak, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 4096 flop/clk x 2.4 GHz, dense bf16 MFMA
PEAK_FP32_VALU_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


# ----------------------------------------------------------------------------
# algorithmic work
# ----------------------------------------------------------------------------

def attended_pairs(w: W.Workload) -> int:
    """(query row, key row) pairs the backward must touch, summed over query heads."""
    if w.form == "selected":
        return w.T1 * w.n1 * w.block_count * w.block_size
    tot = 0
    for s1, s2 in zip(w.seqlens_q, w.seqlens_kv):
        tot += s1 * (s1 + 1) // 2 if w.causal else s1 * s2
    return tot * w.n1


def flops_per_pair(w: W.Workload, gemms=("S", "dP", "dV", "dQ", "dK")) -> int:
    dqk, dv = w.d_qk + w.d_rope, w.d_v
    width = {"S": dqk, "dP": dv, "dV": dv, "dQ": dqk, "dK": dqk, "O": dv}
    return 2 * sum(width[g] for g in gemms)


# library timing name -> (kernel identifier in profiler output, plain or mangled; the source files
# whose text decides its traffic: the kernel's own, and index.hip for the KV-major passes, whose
# work order it computes)
KERNEL_SOURCES = {
    "dense_kv_major": ("dense_kv_kernel", ("dense_kv.hip",)),
    "dense_dq": ("dense_dq_ds_kernel", ("dense_dq.hip",)),
    "dense_dq_recompute": ("dense_dq_kernel", ("attn_q.hip",)),
    "selected_kv_major": ("sel_kv_kernel", ("sel_kv.hip", "index.hip", "share_layout.hpp")),
    "selected_dq_reduce": ("dq_reduce_kernel", ("sel_reduce.hip", "share_layout.hpp")),
    "selected_forward": ("sel_fwd_kv_kernel", ("sel_fwd_kv.hip", "index.hip")),
    "selected_forward_combine": ("sel_fwd_combine_kernel", ("sel_fwd_kv.hip",)),
    "selected_row_stat": ("sel_drow_kv_kernel", ("sel_fwd_kv.hip", "index.hip")),
    "selected_index": ("idx_fill_ordered_kernel", ("index.hip",)),
    "indexer_query_major": ("idx_bwd_kernel", ("indexer.hip",)),
    "indexer_dk_reduce": ("idx_dk_reduce_kernel", ("indexer.hip",)),
    "row_stats": ("preprocess_kernel", ("preprocess.hip",)),
}
CSRC = os.path.join(ROOT, "sparse_attention_backward_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def source_code_only(text: str) -> str:
    """C++ source without its comments and trailing blanks: what a counter record depends on."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(name: str) -> str:
    """sha256 over the code (comments removed) of the kernel's source files and the shared
    headers they include, and over the extra compiler options of the units built from them."""
    import hashlib
    from sparse_attention_backward_amd.build import UNITS
    h = hashlib.sha256()
    files = (*KERNEL_SOURCES[name][1], "common.hpp", "kernels.hpp")
    for f in files:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(source_code_only(fh.read()).encode())
    for unit, src, extra in UNITS:
        if src in files:
            h.update(f"{unit}: {' '.join(extra)}\n".encode())
    return h.hexdigest()


def recorded_counters(name: str, workload: str) -> dict:
    """Counter figures recorded for a kernel on a workload in profiles/counters_<kernel>_<workload>.md
    (lines "- key: value"): HBM traffic per launch (FETCH_SIZE + WRITE_SIZE, each scaled by the copy-kernel
    calibration) and MFMA busy percentage.  Empty when the record is absent or was taken from other kernel
    source (sha256 of the kernel's sources)."""
    path = os.path.join(PROFILES, f"counters_{name}_{workload}.md")
    if not os.path.exists(path) or name not in KERNEL_SOURCES:
        return {}
    vals = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != kernel_source_hash(name):
        return {}
    out = {}
    for k, conv in (("traffic_bytes_per_launch", int), ("mfma_busy_pct", float)):
        try:
            out[k] = conv(vals[k])
        except (KeyError, ValueError):
            pass
    return out


def summarize_counters(dirs, calib_dir=None):
    """Mean counter value per dispatch, per library kernel, from rocprofv3 --pmc CSV output directories;
    with a copy-calibration directory also the FETCH_SIZE / WRITE_SIZE scale factors."""
    import csv
    import glob
    out = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                kn = r["Kernel_Name"]
                for lib_name, (prefix, _) in KERNEL_SOURCES.items():
                    if prefix in kn:
                        acc = out.setdefault(lib_name, {}).setdefault(r["Counter_Name"], [])
                        acc.append(float(r["Counter_Value"]))
    res = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in out.items()}
    if calib_dir:
        cal = {}
        for f in glob.glob(os.path.join(calib_dir, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if "copy" in r["Kernel_Name"].lower() or "elementwise" in r["Kernel_Name"].lower():
                    cal.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        res["_copy_calibration"] = {c: max(v) for c, v in cal.items()}
    return res


# kernel -> the GEMMs it performs (for its roofline point)
KERNEL_GEMMS = {
    "dense_kv_major": ("S", "dP", "dV", "dK"),
    "dense_dq": ("dQ",),
    "dense_dq_recompute": ("S", "dP", "dQ"),
    "selected_kv_major": ("S", "dP", "dV", "dK", "dQ"),
    "dense_fp32": ("S", "dP", "dV", "dQ", "dK", "S", "dP"),
    "selected_forward": ("S", "O"),
}


# ----------------------------------------------------------------------------
# input preparation (GPU, fp32 torch; not timed)
# ----------------------------------------------------------------------------

def _cat(a, b):
    return a if b is None else torch.cat([a, b], dim=-1)


@torch.no_grad()
def gpu_forward(w: W.Workload, x):
    """O (workload dtype) and [T1, N1, 8] fp32 softmax max / sum of the forward: for the dense
    workloads a plain fp32 torch forward per sequence, for the selected ones the library's
    attn_fwd_selected."""
    dev = x["query"].device
    T1 = w.T1
    G = w.G
    if w.form == "dense":
        O = torch.zeros((T1, w.n1, w.d_v), device=dev, dtype=torch.float32)
        m = torch.full((T1, w.n1), -math.inf, device=dev)
        l = torch.zeros((T1, w.n1), device=dev)
        Q = _cat(x["query"], x["query_rope"]).float()
        K = _cat(x["key"], x["key_rope"]).float()
        V = x["value"].float()
        cq, ck = w.cu_q, w.cu_kv
        for b in range(w.batch):
            qs, qe, ks, ke = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
            if qe == qs or ke == ks:
                continue
            Qb = Q[qs:qe].transpose(0, 1).contiguous()                                # [N1, S1, D]
            Kb = K[ks:ke].repeat_interleave(G, dim=1).transpose(0, 1).contiguous()   # [N1, S2, D]
            Vb = V[ks:ke].repeat_interleave(G, dim=1).transpose(0, 1).contiguous()
            S = torch.bmm(Qb, Kb.transpose(1, 2).contiguous()) * w.scale
            if w.causal:
                mask = torch.ones(qe - qs, ke - ks, dtype=torch.bool, device=dev).triu(1)
                S.masked_fill_(mask, -math.inf)
            mb = S.amax(dim=-1)
            P = torch.exp(S - mb[..., None])
            lb = P.sum(-1)
            O[qs:qe] = torch.bmm(P / lb[..., None], Vb).transpose(0, 1)
            m[qs:qe] = mb.transpose(0, 1)
            l[qs:qe] = lb.transpose(0, 1)
            del S, P
    else:
        # the library's own selected forward (one launch; its parity is tested against the oracle)
        prob = sab.Problem.selected(w.cu_q, w.cu_kv, w.n1, w.n2, w.d_qk, w.d_v, w.scale, w.block_size,
                                    w.block_count, dtype=w.dtype, forward=True)
        out, smax, ssum = sab.selected_forward(prob, x["query"], x["key"], x["value"], x["topk"])
        torch.cuda.synchronize()
        return out, smax, ssum
    smax = m[..., None].expand(T1, w.n1, 8).contiguous()
    ssum = l[..., None].expand(T1, w.n1, 8).contiguous()
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return O.to(dt), smax, ssum


# ----------------------------------------------------------------------------
# timed run
# ----------------------------------------------------------------------------

def make_problem(w: W.Workload, deterministic=False, window_tokens=0):
    if w.form == "dense":
        return sab.Problem.dense(w.cu_q, w.cu_kv, w.n1, w.n2, w.d_qk, w.d_v, w.scale, causal=w.causal,
                                 d_rope=w.d_rope, dtype=w.dtype, deterministic=deterministic)
    return sab.Problem.selected(w.cu_q, w.cu_kv, w.n1, w.n2, w.d_qk, w.d_v, w.scale, w.block_size,
                                w.block_count, deterministic=deterministic, window_tokens=window_tokens)


def run_workload(w: W.Workload, steps: int, warmup: int, deterministic=False, window_tokens=0, prewarm_ms=300.0,
                 with_out=True):
    """Time `steps` complete calls after a clock pre-warm (calls repeated until `prewarm_ms` of GPU time
    have passed) and `warmup` untimed calls.  Returns the inputs, ms per call, the library's per-kernel
    totals over the timed calls, and the pre-warm actually spent."""
    dev = torch.device("cuda", 0)
    x = W.make_inputs(w, device=dev, backend="torch")
    o, smax, ssum = gpu_forward(w, x)
    if not with_out:  # the selected call without attentionOut (the row statistic from the gathered rows)
        o = None
    prob = make_problem(w, deterministic, window_tokens)
    if w.form == "dense":
        outs = [torch.empty_like(x["query"]), torch.empty_like(x["query_rope"]) if w.d_rope else None,
                torch.empty_like(x["key"]), torch.empty_like(x["key_rope"]) if w.d_rope else None,
                torch.empty_like(x["value"])]
    else:
        outs = [torch.empty_like(x["query"]), torch.empty_like(x["key"]), torch.empty_like(x["value"])]
    ws = torch.empty(max(1, sab.attn_bwd_workspace_size(prob)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        if w.form == "dense":
            sab.attn_bwd_dense_varlen(prob, x["query"], x["query_rope"], x["key"], x["key_rope"], x["value"], o,
                                      x["dy"], smax, ssum, *outs, ws, stream=stream)
        else:
            sab.attn_bwd_selected(prob, x["query"], x["key"], x["value"], o, x["dy"], smax, ssum, x["topk"],
                                  *outs, ws, stream=stream)

    # The GPU raises its clock over the first tens of milliseconds of sustained work: repeat the
    # call until prewarm_ms have passed (measured with events, in batches), then the warmup calls.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    spent, batch = 0.0, 1
    while spent < prewarm_ms:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(batch):
            step()
        b.record(stream)
        b.synchronize()
        spent += a.elapsed_time(b)
        batch = min(batch * 2, 64)
        if time.perf_counter() - t0 > 60:
            break
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    sab.attn_bwd_profile_reset()
    sab.attn_bwd_profiling(True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    sab.attn_bwd_profiling(False)
    ms = start.elapsed_time(end) / steps
    kernels = sab.attn_bwd_profile_read()
    return x, ms, kernels, spent


def algorithmic_bytes(w: W.Workload) -> int:
    """HBM bytes the call must move at the least: every input read once and every output written once."""
    e = 2 if w.dtype == "bf16" else 4
    dqk = w.d_qk + w.d_rope
    by = w.T1 * w.n1 * dqk * e * 2                      # Q (+ queryRope) in, dQ (+ dqRope) out
    by += w.T2 * w.n2 * (dqk + w.d_v) * e * 2           # K (+ keyRope), V in; dK (+ dkRope), dV out
    by += 2 * w.T1 * w.n1 * w.d_v * e                   # O, dY
    by += 2 * w.T1 * w.n1 * 8 * 4                       # softmaxMax, softmaxSum [T1, N1, 8] fp32
    if w.form == "selected":
        by += w.T1 * w.n2 * w.block_count * 4           # topkIndices
    return by


def roofline_for(w: W.Workload, kernels: dict, steps: int, call_ms: float):
    """Roofline point of the dominant kernel (largest time per call): its algorithmic GEMM flops per call
    (attended pairs x 2 x the widths of the GEMMs it performs) over its time per call, against the bf16
    MFMA peak (fp32 config: against the fp32 vector peak).  `hbm_view`: the call's algorithmic bytes
    (inputs read and outputs written once) over the call time, against 8 TB/s.  `traffic`: HBM bytes of
    the kernel per launch from the recorded rocprofv3 counters (null when absent or stale)."""
    name = max(kernels, key=lambda k: kernels[k][0])
    tot_ms, n = kernels[name]
    per_call_ms = tot_ms / max(steps, 1)
    launches = n / max(steps, 1)
    gemms = KERNEL_GEMMS.get(name)
    rec = recorded_counters(name, w.name)
    ab_bytes = algorithmic_bytes(w)
    out = {"kernel": name, "avg_ms": tot_ms / max(n, 1), "launches_per_call": launches,
           "ms_per_call": per_call_ms}
    if gemms is None:
        out.update({"bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": None})
    else:
        fl = attended_pairs(w) * flops_per_pair(w, gemms)
        achieved = fl / (per_call_ms * 1e-3) / 1e12
        if w.dtype == "fp32":
            out.update({"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                        "frac": achieved / PEAK_FP32_VALU_TFLOPS})
        else:
            out.update({"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": achieved / PEAK_BF16_TFLOPS})
        out["flop_per_call"] = fl
        out["flop_per_launch"] = fl / max(launches, 1e-9)
    traffic = rec.get("traffic_bytes_per_launch")
    out["traffic"] = traffic
    if traffic is not None:
        out["traffic_per_call"] = traffic * launches
        out["traffic_vs_algorithmic_call_bytes"] = traffic * launches / ab_bytes
    if "mfma_busy_pct" in rec:
        out["mfma_busy_pct_counter"] = rec["mfma_busy_pct"]
    out["hbm_view"] = {"algorithmic_bytes_per_call": ab_bytes,
                       "achieved_gbs": ab_bytes / (call_ms * 1e-3) / 1e9,
                       "frac": ab_bytes / (call_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    return out


def progress(rec: dict) -> None:
    """One line on stderr as each measured record completes."""
    print(f"[bench] {rec.get('workload')} {rec.get('pass', 'backward')}: {rec.get('ms_per_step')} ms per call",
          file=sys.stderr, flush=True)


def measure(wl: int, steps: int, warmup: int, deterministic=False, window_tokens=0, prewarm_ms=300.0, with_out=True):
    """One bench record for workload `wl`: value, timing, roofline and per-kernel times."""
    w = W.config(wl)
    x, ms, kernels, spent = run_workload(w, steps, warmup, deterministic, window_tokens, prewarm_ms, with_out)
    total_flops = attended_pairs(w) * flops_per_pair(w)
    value = total_flops / (ms * 1e-3) / 1e12
    rec = {
        "workload": w.name,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "ms_per_step": round(ms, 4),
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "config": {"workload": w.name, "form": w.form, "seqlens": list(w.seqlens_q), "n1": w.n1, "n2": w.n2,
                   "d_qk": w.d_qk, "d_rope": w.d_rope, "d_v": w.d_v, "causal": w.causal,
                   "block_size": w.block_size, "block_count": w.block_count, "index_dist": w.index_dist,
                   "deterministic": bool(deterministic), "window_tokens": int(window_tokens),
                   "attention_out": bool(with_out),
                   "algorithmic_tflop_per_step": total_flops / 1e12},
        "roofline": roofline_for(w, kernels, steps, ms),
        "kernels_ms_per_call": {k: round(v[0] / steps, 4) for k, v in kernels.items()},
        "kernel_launches_per_call": {k: v[1] / steps for k, v in kernels.items()},
        "prewarm_ms": round(spent, 1),
    }
    progress(rec)
    return w, x, rec


# ----------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample of the same workload
# ----------------------------------------------------------------------------

def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        return max(n) if n else os.cpu_count()
    except Exception:
        return os.cpu_count()


def cpu_baseline(w: W.Workload, x, budget_s=12.0):
    import oracle as O
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    G = w.G
    done_flops, done_units, elapsed = 0, [], 0.0
    if w.form == "dense":
        # units: (sequence, KV head) groups, shortest sequence first
        order = sorted(range(w.batch), key=lambda b: w.seqlens_q[b])
        for b in order:
            qs, qe, ks, ke = (int(w.cu_q[b]), int(w.cu_q[b + 1]), int(w.cu_kv[b]), int(w.cu_kv[b + 1]))
            for kvh in range(w.n2):
                hs = slice(kvh * G, (kvh + 1) * G)
                sub = lambda t, h: None if t is None else f64(t[qs:qe, h])  # noqa: E731
                args = (sub(x["query"], hs), f64(x["key"][ks:ke, kvh:kvh + 1]), f64(x["value"][ks:ke, kvh:kvh + 1]),
                        sub(x["dy"], hs), np.array([0, qe - qs]), np.array([0, ke - ks]), G, 1, w.scale, w.causal,
                        sub(x["query_rope"], hs), None if x["key_rope"] is None else f64(x["key_rope"][ks:ke, kvh:kvh + 1]))
                t0 = time.perf_counter()
                O.backward_dense(*args)
                elapsed += time.perf_counter() - t0
                s1, s2 = qe - qs, ke - ks
                pairs = (s1 * (s1 + 1) // 2 if w.causal else s1 * s2) * G
                done_flops += pairs * flops_per_pair(w)
                done_units.append(f"seq{b}/kvhead{kvh}")
                if elapsed >= budget_s:
                    break
            if elapsed >= budget_s:
                break
        sample = f"{len(done_units)} of {w.batch * w.n2} (sequence, KV-head group) units ({done_units[0]}..{done_units[-1]})"
    else:
        b = 0
        qs, qe, ks, ke = (int(w.cu_q[b]), int(w.cu_q[b + 1]), int(w.cu_kv[b]), int(w.cu_kv[b + 1]))
        Kc, Vc = f64(x["key"][ks:ke]), f64(x["value"][ks:ke])
        ntok, step_t = 0, 16
        while elapsed < budget_s and qs + ntok < qe:
            t0, t1 = qs + ntok, min(qe, qs + ntok + step_t)
            a = time.perf_counter()
            O.backward_selected(f64(x["query"][t0:t1]), Kc, Vc, f64(x["dy"][t0:t1]), x["topk"][t0:t1].cpu().numpy(),
                                np.array([0, t1 - t0]), np.array([0, ke - ks]), w.n1, w.n2, w.scale, w.block_size)
            elapsed += time.perf_counter() - a
            ntok += t1 - t0
        done_flops = ntok * w.n1 * w.block_count * w.block_size * flops_per_pair(w)
        sample = f"first {ntok} query tokens of sequence 0 (all heads)"
    return {"value": done_flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": sample, "seconds": round(elapsed, 2), "host_cpus": os.cpu_count()}


# ----------------------------------------------------------------------------

def measure_forward(wl: int, steps: int, warmup: int, prewarm_ms=300.0):
    """The selected forward (attn_fwd_selected) on workload `wl`: its own record, with the two
    GEMMs S and O = P V (2 (D_qk + D_v) flop per attended pair) as the algorithmic work."""
    w = W.config(wl)
    dev = torch.device("cuda", 0)
    x = W.make_inputs(w, device=dev, backend="torch")
    prob = sab.Problem.selected(w.cu_q, w.cu_kv, w.n1, w.n2, w.d_qk, w.d_v, w.scale, w.block_size,
                                w.block_count, dtype=w.dtype, forward=True)
    ws = torch.empty(max(1, sab.attn_bwd_workspace_size(prob)), dtype=torch.uint8, device=dev)
    out = torch.empty((w.T1, w.n1, w.d_v), dtype=x["query"].dtype, device=dev)
    smax = torch.empty((w.T1, w.n1, 8), dtype=torch.float32, device=dev)
    ssum = torch.empty_like(smax)
    stream = torch.cuda.current_stream()

    def step():
        sab.attn_fwd_selected(prob, x["query"], x["key"], x["value"], x["topk"], out, smax, ssum, ws, stream=stream)

    torch.cuda.synchronize()
    spent, t0 = 0.0, time.perf_counter()
    while spent < prewarm_ms and time.perf_counter() - t0 < 60:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        b.synchronize()
        spent += a.elapsed_time(b)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    sab.attn_bwd_profile_reset()
    sab.attn_bwd_profiling(True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    sab.attn_bwd_profiling(False)
    ms = a.elapsed_time(b) / steps
    kernels = sab.attn_bwd_profile_read()
    fl = attended_pairs(w) * flops_per_pair(w, ("S", "O"))
    tot_ms, n = kernels["selected_forward"]
    kms = tot_ms / steps
    launches = n / max(steps, 1)
    # what the KV-major pass moves per (token, KV head, slot): the G query rows gathered and the
    # entry's partial (G d_v elements + G (m_b, l_b)) written
    e = 2 if w.dtype != "fp32" else 4
    gather = w.T1 * w.n2 * w.block_count * w.G * (w.d_qk * e + w.d_v * e + 8)
    rec = {"workload": w.name, "pass": "forward", "value": round(fl / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
           "ms_per_step": round(ms, 4), "steps": steps,
           "pct_bf16_peak": round(100.0 * fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
           "roofline": {"kernel": "selected_forward", "bound": "mfma", "avg_ms": tot_ms / max(n, 1),
                        "achieved": fl / (kms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": fl / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "flop_per_launch": fl / max(launches, 1e-9),
                        "launches_per_call": launches,
                        "traffic": recorded_counters("selected_forward", w.name).get("traffic_bytes_per_launch"),
                        "kv_pass_bytes_per_call": gather, "kv_pass_gbs": gather / (kms * 1e-3) / 1e9},
           "kernels_ms_per_call": {k: round(v[0] / steps, 4) for k, v in kernels.items()},
           "prewarm_ms": round(spent, 1)}
    del x, out, smax, ssum, ws
    torch.cuda.empty_cache()
    progress(rec)
    return rec


def indexer_record_name(w, dk_atomic: bool) -> str:
    """Workload name of the indexer's counter records: the two dK modes run different kernels."""
    return f"{w.name}-{'atomic' if dk_atomic else 'ordered'}"


def measure_indexer(dk_atomic: bool, steps: int, warmup: int, prewarm_ms=300.0):
    """The lightning-indexer backward (attn_bwd_indexer) on its 8K workload: three GEMMs per
    (token, key head, selected key) -- S = Q K^T, dQ = R K, dK shares = R^T Q -- i.e.
    2 x 3 x G x D flop per (token, key head, slot)."""
    w = W.indexer_config()
    dev = torch.device("cuda", 0)
    x = W.make_indexer_inputs(w, device=dev, backend="torch")
    prob = sab.Problem.indexer(w.cu_q, w.cu_kv, w.n1, w.n2, w.topk, d=w.d, dk_atomic=dk_atomic)
    ws = torch.empty(max(1, sab.attn_bwd_workspace_size(prob)), dtype=torch.uint8, device=dev)
    dq, dk, dw = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["weights"])
    stream = torch.cuda.current_stream()

    def step():
        sab.attn_bwd_indexer(prob, x["q"], x["k"], x["weights"], x["dy"], x["indices"], dq, dk, dw, ws, stream=stream)

    torch.cuda.synchronize()
    spent, t0 = 0.0, time.perf_counter()
    while spent < prewarm_ms and time.perf_counter() - t0 < 60:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        b.synchronize()
        spent += a.elapsed_time(b)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    sab.attn_bwd_profile_reset()
    sab.attn_bwd_profiling(True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    sab.attn_bwd_profiling(False)
    ms = a.elapsed_time(b) / steps
    kernels = sab.attn_bwd_profile_read()
    fl = w.T1 * w.n1 * w.topk * w.d * 6
    tot_ms, n = kernels["indexer_query_major"]
    kms = tot_ms / steps
    rec = {"workload": w.name, "pass": "indexer backward", "dk": "fp32 atomics" if dk_atomic else "ordered sums",
           "value": round(fl / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "ms_per_step": round(ms, 4),
           "steps": steps, "pct_bf16_peak": round(100.0 * fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
           "roofline": {"kernel": "indexer_query_major", "bound": "mfma", "avg_ms": tot_ms / max(n, 1),
                        "launches_per_call": n / max(steps, 1),
                        "achieved": fl / (kms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": fl / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "flop_per_call": fl,
                        "traffic": recorded_counters("indexer_query_major", indexer_record_name(w, dk_atomic))
                        .get("traffic_bytes_per_launch")},
           "kernels_ms_per_call": {k: round(v[0] / steps, 4) for k, v in kernels.items()},
           "prewarm_ms": round(spent, 1)}
    del x, ws, dq, dk, dw
    torch.cuda.empty_cache()
    progress(rec)
    return rec


EXTRA_RUNS = ((2, False), (3, False), (4, False), (4, True))  # (workload, deterministic) beside the headline
NO_OUT_RUNS = (3,)  # the selected backward without attentionOut, measured on these workloads
FORWARD_RUNS = (5, 3)  # selected forward measured on these workloads


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prewarm-ms", type=float, default=300.0,
                    help="GPU time spent repeating the call before the warmup calls (clock ramp)")
    ap.add_argument("--workload", type=int, default=5,
                    help="headline workload 1..5 (default 5: selected bf16 at S = 128K, the largest)")
    ap.add_argument("--deterministic", action="store_true")
    ap.add_argument("--window-tokens", type=int, default=0, help="selected: query tokens per window (0 automatic)")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads' lines")
    ap.add_argument("--indexer-only", action="store_true",
                    help="only the lightning-indexer backward lines (for profiling runs)")
    ap.add_argument("--indexer-mode", choices=("both", "ordered", "atomic"), default="both",
                    help="with --indexer-only: which dK mode(s) to run")
    ap.add_argument("--forward-only", action="store_true",
                    help="only the selected forward lines (for profiling runs)")
    ap.add_argument("--forward-workload", type=int, default=0,
                    help="with --forward-only: this workload alone (0: all forward workloads)")
    ap.add_argument("--no-out", action="store_true",
                    help="selected headline without attentionOut (the row statistic from the gathered rows)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB 5 times (counter calibration)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="print per-kernel mean counters of rocprofv3 --pmc output directories and exit "
                         "(with --calibration DIR: also the copy kernel's FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--calibration", metavar="DIR")
    ap.add_argument("--source-hash", metavar="KERNEL", help="print the kernel source hash used by counter records")
    args = ap.parse_args(argv)
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters, args.calibration), indent=1))
        return 0
    if args.source_hash:
        print(kernel_source_hash(args.source_hash))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)
        return 0

    if args.forward_only:
        wls = (args.forward_workload,) if args.forward_workload else FORWARD_RUNS
        print(json.dumps([measure_forward(wl, args.steps, args.warmup, args.prewarm_ms) for wl in wls]), flush=True)
        return 0
    if args.indexer_only:
        modes = {"both": (False, True), "ordered": (False,), "atomic": (True,)}[args.indexer_mode]
        print(json.dumps([measure_indexer(a, args.steps, args.warmup, args.prewarm_ms) for a in modes]), flush=True)
        return 0
    w, x, rec = measure(args.workload, args.steps, args.warmup, args.deterministic, args.window_tokens,
                        args.prewarm_ms, with_out=not args.no_out)
    line = {
        "metric": METRIC,
        "value": rec["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec["dtype"],
        "data": "synthetic",
        "config": rec["config"],
        "pct_bf16_peak": rec["pct_bf16_peak"],
        "roofline": rec["roofline"],
        "kernels_ms_per_call": rec["kernels_ms_per_call"],
        "kernel_launches_per_call": rec["kernel_launches_per_call"],
        "prewarm_ms": rec["prewarm_ms"],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, x)
    del x
    torch.cuda.empty_cache()
    if not args.no_extra:
        extra = []
        for wl, det in EXTRA_RUNS:
            if wl == args.workload and det == args.deterministic:
                continue
            # the dense workload's calls are short: time more of them
            k = args.steps * 10 if W.config(wl).form == "dense" else args.steps
            _, xe, re_ = measure(wl, k, args.warmup, det, 0, args.prewarm_ms)
            re_["steps"] = k
            extra.append(re_)
            del xe
            torch.cuda.empty_cache()
        for wl in NO_OUT_RUNS:
            _, xe, re_ = measure(wl, args.steps, args.warmup, False, 0, args.prewarm_ms, with_out=False)
            re_["pass"] = "backward without attentionOut"
            extra.append(re_)
            del xe
            torch.cuda.empty_cache()
        for wl in FORWARD_RUNS:
            extra.append(measure_forward(wl, max(3, args.steps // 2), args.warmup, args.prewarm_ms))
        for atomic in (False, True):
            extra.append(measure_indexer(atomic, args.steps, args.warmup, args.prewarm_ms))
        line["extra"] = extra
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
