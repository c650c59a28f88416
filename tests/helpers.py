"""Shared helpers for the parity tests: oracle-side inputs, GPU calls, tolerances.

Inputs come from the seeded generators in ``workloads``; O and the softmax
statistics come from the float64 oracle forward (never from the GPU path).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import workloads as W

# Tolerances per output tensor.
BF16_REL_L2 = 1e-2
BF16_MAX_ABS = 2e-2   # times max |ref|
FP32_REL_L2 = 1e-4
# fp16 (no bar is stated for it): the bf16 bar scaled by the ratio of the unit roundoffs,
# 2^-11 / 2^-8, with a factor 2 for the P and dS operands rounded to fp16 before their products
FP16_REL_L2 = 2.5e-3
FP16_MAX_ABS = 5e-3
# A reference of exact zeros (e.g. rows that see a single key: P = 1, dS = P (dP - D) = 0) is
# met within this absolute bound: the kernels form dP and D = rowsum(dY O) as two fp32 dot
# products of magnitude ~10 whose rounding leaves ~1e-6 in dS.
ZERO_ABS = 1e-5


def f64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def assert_close(name, got, ref, dtype):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    if ref.size == 0:
        return
    nref = np.linalg.norm(ref)
    err = np.linalg.norm(got - ref)
    rel = err / nref if nref > 0 else err
    mx = np.abs(got - ref).max()
    mref = np.abs(ref).max()
    if dtype == "fp32":
        assert rel <= FP32_REL_L2 or (nref == 0 and mx <= ZERO_ABS), f"{name}: rel L2 {rel:.3e} > {FP32_REL_L2}"
    elif dtype == "fp16":
        if nref == 0:
            assert mx <= ZERO_ABS, f"{name}: expected zeros, max |x| = {mx:.3e}"
            return
        assert rel <= FP16_REL_L2, f"{name}: rel L2 {rel:.3e} > {FP16_REL_L2}"
        assert mx <= FP16_MAX_ABS * mref, f"{name}: max abs {mx:.3e} > {FP16_MAX_ABS} * {mref:.3e}"
    else:
        if nref == 0:
            assert mx <= ZERO_ABS, f"{name}: expected zeros, max |x| = {mx:.3e}"
            return
        assert rel <= BF16_REL_L2, f"{name}: rel L2 {rel:.3e} > {BF16_REL_L2}"
        assert mx <= BF16_MAX_ABS * mref, f"{name}: max abs {mx:.3e} > {BF16_MAX_ABS} * {mref:.3e}"


def mask_of(w: W.Workload):
    """The oracle's mask argument for a dense workload: False, True (causal, equal lengths,
    top-left) or a BandMask (causal aligned either way, or a window)."""
    align = "bottom_right" if w.mask_align else "top_left"
    if w.band is not None:
        return O.BandMask(w.band[0], w.band[1], align)
    if w.causal and (w.mask_align or w.seqlens_q != w.seqlens_kv):
        return O.BandMask(float("inf"), 0, align)
    return w.causal


def oracle_forward(w: W.Workload, x):
    """O (cast to the workload dtype) and the [T, N, 8] statistics, from the oracle."""
    if w.form == "dense":
        o, m, l = O.forward_dense(f64(x["query"]), f64(x["key"]), f64(x["value"]), w.cu_q, w.cu_kv, w.n1, w.n2,
                                  w.scale, mask_of(w), f64(x["query_rope"]), f64(x["key_rope"]))
    else:
        o, m, l = O.forward_selected(f64(x["query"]), f64(x["key"]), f64(x["value"]), x["topk"].numpy(),
                                     w.cu_q, w.cu_kv, w.n1, w.n2, w.scale, w.block_size)
    smax, ssum = O.stats_tensor(m, l)
    return W.cast(o, w.dtype), torch.from_numpy(smax), torch.from_numpy(ssum)


def oracle_backward(w: W.Workload, x):
    if w.form == "dense":
        dq, dqr, dk, dkr, dv = O.backward_dense(f64(x["query"]), f64(x["key"]), f64(x["value"]), f64(x["dy"]),
                                                w.cu_q, w.cu_kv, w.n1, w.n2, w.scale, mask_of(w),
                                                f64(x["query_rope"]), f64(x["key_rope"]))
        return {"dq": dq, "dq_rope": dqr if w.d_rope else None, "dk": dk, "dk_rope": dkr if w.d_rope else None,
                "dv": dv}
    dq, dk, dv = O.backward_selected(f64(x["query"]), f64(x["key"]), f64(x["value"]), f64(x["dy"]),
                                     x["topk"].numpy(), w.cu_q, w.cu_kv, w.n1, w.n2, w.scale, w.block_size)
    return {"dq": dq, "dk": dk, "dv": dv}


def problem_for(w: W.Workload, deterministic=None, dq_mode=0, window_tokens=0):
    import sparse_attention_backward_amd as sab
    det = w.deterministic if deterministic is None else deterministic
    if w.form == "dense":
        return sab.Problem.dense(w.cu_q, w.cu_kv, w.n1, w.n2, w.d_qk, w.d_v, w.scale, causal=w.causal,
                                 d_rope=w.d_rope, dtype=w.dtype, deterministic=det, dq_mode=dq_mode,
                                 align=w.mask_align, band=w.band)
    return sab.Problem.selected(w.cu_q, w.cu_kv, w.n1, w.n2, w.d_qk, w.d_v, w.scale, w.block_size, w.block_count,
                                deterministic=det, window_tokens=window_tokens, dtype=w.dtype)


def gpu_backward(w: W.Workload, x, o, smax, ssum, device="cuda", deterministic=None, dq_mode=0, window_tokens=0):
    """Run the library on the GPU; returns the output tensors (on the device).  o = None: the
    selected call without attentionOut."""
    import sparse_attention_backward_amd as sab
    dev = lambda t: None if t is None else t.to(device).contiguous()  # noqa: E731
    prob = problem_for(w, deterministic, dq_mode, window_tokens)
    if w.form == "dense":
        outs = sab.dense_backward(prob, dev(x["query"]), dev(x["query_rope"]), dev(x["key"]), dev(x["key_rope"]),
                                  dev(x["value"]), dev(o), dev(x["dy"]), dev(smax), dev(ssum))
        torch.cuda.synchronize()
        names = ("dq", "dq_rope", "dk", "dk_rope", "dv")
    else:
        outs = sab.selected_backward(prob, dev(x["query"]), dev(x["key"]), dev(x["value"]), dev(o), dev(x["dy"]),
                                     dev(smax), dev(ssum), dev(x["topk"]))
        torch.cuda.synchronize()
        names = ("dq", "dk", "dv")
    return {n: (None if t is None else t) for n, t in zip(names, outs)}


def assert_rows_close(name, got, ref, dtype, frac=None):
    """Row by row ([T, N, D] -> one row per (token, head)): every row's error norm within a
    fraction of that row's norm, or of the median row norm for rows near zero.  A row that
    lost or gained a whole term of its sum (a block's share of dQ) fails here even when the
    tensor-wide norms hide it."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(got)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    if ref.size == 0:
        return
    frac = frac if frac is not None else {"fp32": 1e-3, "fp16": 1e-2}.get(dtype, 4e-2)
    rn = np.linalg.norm(ref, axis=1)
    floor = np.median(rn[rn > 0]) if (rn > 0).any() else 0.0
    err = np.linalg.norm(got - ref, axis=1)
    bad = np.nonzero(err > frac * np.maximum(rn, floor) + ZERO_ABS)[0]
    assert bad.size == 0, (f"{name}: {bad.size} rows off, first row {bad[0]}: error {err[bad[0]]:.3e}, "
                           f"row norm {rn[bad[0]]:.3e}")


def check_against_oracle(w: W.Workload, got, ref):
    for name, r in ref.items():
        if r is None:
            assert got.get(name) is None
            continue
        assert_close(f"{w.name}:{name}", f64(got[name]), r, w.dtype)
        if name == "dq":
            assert_rows_close(f"{w.name}:{name} rows", f64(got[name]), r, w.dtype)
