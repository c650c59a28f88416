"""Seeded synthetic inputs for the attention-backward workloads.

This module holds shapes, random draws and dtype casts only -- none of the
attention arithmetic.  Both the float64 oracle (through the tests) and the GPU
library consume what it produces.

Draws (all seeded):
* sequence lengths: ``numpy.random.default_rng(seed)``;
* Q, K, V, dY: i.i.d. N(0, 1), cast to the workload dtype (bf16 round to
  nearest even, or fp32);
* topkIndices [T1, N2, cnt] int32, per (token, KV head) row, ``cnt`` distinct
  block ids of the token's own sequence, either uniform (prefix of a random
  permutation) or Zipf-skewed towards low ids (Gumbel-top-k sampling without
  replacement with weights (id + 1) ** -s), kept in sampled order.

Two backends draw the same distributions: ``numpy`` (PCG64, CPU; exact
reproducibility for small cases) and ``torch`` (the device's Philox stream;
used at full sizes where CPU draws would take minutes).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

__all__ = ["Workload", "config", "CONFIGS", "make_inputs", "cast", "small_dense", "small_selected",
           "IndexerWorkload", "indexer_config", "small_indexer", "make_indexer_inputs"]


@dataclass(frozen=True)
class Workload:
    name: str
    form: str                      # "dense" or "selected"
    dtype: str                     # "bf16", "fp16" or "fp32"
    seqlens_q: tuple
    seqlens_kv: tuple
    n1: int
    n2: int
    d_qk: int                      # query / key head dim (main part)
    d_v: int
    scale: float
    d_rope: int = 0                # dense only: queryRope / keyRope head dim
    causal: bool = False
    mask_align: int = 0            # dense masks: 0 top-left, 1 bottom-right alignment
    band: tuple = None             # dense: (pre_tokens, next_tokens) window, or None
    block_size: int = 0            # selected only
    block_count: int = 0
    index_dist: str = "uniform"    # "uniform" or "zipf"
    zipf_s: float = 1.1
    seed: int = 0
    deterministic: bool = False
    notes: str = field(default="", compare=False)

    @property
    def batch(self):
        return len(self.seqlens_q)

    @property
    def T1(self):
        return int(sum(self.seqlens_q))

    @property
    def T2(self):
        return int(sum(self.seqlens_kv))

    @property
    def G(self):
        return self.n1 // self.n2

    @property
    def cu_q(self):
        return np.concatenate([[0], np.cumsum(self.seqlens_q)]).astype(np.int64)

    @property
    def cu_kv(self):
        return np.concatenate([[0], np.cumsum(self.seqlens_kv)]).astype(np.int64)

    def with_(self, **kw):
        return replace(self, **kw)


def config(i: int) -> Workload:
    """The five workloads, with their seeded sequence lengths."""
    if i == 1:
        return Workload("dense-fp32-causal-T160", "dense", "fp32", (64, 96), (64, 96), 2, 2, 64, 64,
                        1.0 / 8.0, causal=True, seed=1)
    if i == 2:
        lens = tuple(int(x) for x in np.random.default_rng(2).integers(512, 4097, 4))
        return Workload("dense-bf16-causal-rope-B4-GQA4", "dense", "bf16", lens, lens, 32, 8, 128, 128,
                        1.0 / math.sqrt(192.0), d_rope=64, causal=True, seed=2)
    if i == 3:
        return Workload("selected-bf16-S32K-bs64-cnt16", "selected", "bf16", (32768,), (32768,), 64, 4,
                        192, 128, 1.0 / math.sqrt(192.0), block_size=64, block_count=16, seed=3)
    if i == 4:
        lens = tuple(int(128 * x) for x in np.random.default_rng(4).integers(32, 129, 8))
        return Workload("selected-bf16-varlen-B8-bs128-cnt32-zipf", "selected", "bf16", lens, lens, 32, 2,
                        192, 128, 1.0 / math.sqrt(192.0), block_size=128, block_count=32,
                        index_dist="zipf", zipf_s=1.1, seed=4)
    if i == 5:
        return Workload("selected-bf16-S128K-bs64-cnt32", "selected", "bf16", (131072,), (131072,), 64, 4,
                        192, 128, 1.0 / math.sqrt(192.0), block_size=64, block_count=32, seed=5)
    raise ValueError(f"no workload {i}")


CONFIGS = (1, 2, 3, 4, 5)


def small_dense(seqlens=(200, 130), n1=8, n2=2, d_qk=128, d_rope=64, d_v=128, dtype="bf16",
                causal=True, seed=11, scale=None, seqlens_kv=None, mask_align=0, band=None):
    """A multi-tile dense case with a ragged tail, small enough for the oracle."""
    d = d_qk + d_rope
    kv = tuple(seqlens_kv) if seqlens_kv is not None else tuple(seqlens)
    return Workload(f"dense-small-{dtype}", "dense", dtype, tuple(seqlens), kv, n1, n2,
                    d_qk, d_v, scale if scale is not None else 1.0 / math.sqrt(d), d_rope=d_rope,
                    causal=causal, mask_align=mask_align, band=band, seed=seed)


def small_selected(seqlens=(256, 384), n1=32, n2=2, d_qk=192, d_v=128, block_size=64,
                   block_count=3, index_dist="uniform", seed=13, seqlens_kv=None, dtype="bf16"):
    """A multi-block selected case small enough for the oracle."""
    kv = tuple(seqlens_kv) if seqlens_kv is not None else tuple(seqlens)
    return Workload(f"selected-small-{dtype}", "selected", dtype, tuple(seqlens), kv, n1, n2, d_qk, d_v,
                    1.0 / math.sqrt(d_qk), block_size=block_size, block_count=block_count,
                    index_dist=index_dist, seed=seed)


# ----------------------------------------------------------------------------
# dtype casts
# ----------------------------------------------------------------------------

_TORCH_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def cast(x, dtype: str, device="cpu"):
    """float64 / float32 array or tensor -> torch tensor of the workload dtype
    (round to nearest even)."""
    t = torch.as_tensor(x)
    if t.dtype == torch.float64 and dtype in ("bf16", "fp16"):
        t = t.to(torch.float32)
    return t.to(device=device, dtype=_TORCH_DTYPES[dtype]).contiguous()


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------

def _normal_np(rng, shape):
    return rng.standard_normal(shape)


def _normal_torch(gen, shape, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _topk_rows_np(rng, rows, nblk, cnt, dist, s):
    """cnt distinct ids in [0, nblk) per row, in sampled order."""
    u = np.clip(rng.random((rows, nblk)), 1e-300, None)
    if dist == "uniform":
        keys = u                                                 # random permutation
    else:
        logw = -s * np.log(np.arange(nblk) + 1.0)
        keys = logw[None, :] - np.log(-np.log(u))                # Gumbel-top-k
    return np.argsort(-keys, axis=1, kind="stable")[:, :cnt].astype(np.int32)


def _topk_rows_torch(gen, rows, nblk, cnt, dist, s, device, chunk=8192):
    """Same distributions as _topk_rows_np, drawn from a torch generator."""
    out = torch.empty((rows, cnt), dtype=torch.int32, device=device)
    logw = -s * torch.log(torch.arange(nblk, device=device, dtype=torch.float32) + 1.0)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        u = torch.rand((r1 - r0, nblk), generator=gen, device=device, dtype=torch.float32).clamp_min(1e-30)
        keys = u if dist == "uniform" else logw[None, :] - torch.log(-torch.log(u))
        out[r0:r1] = torch.argsort(-keys, dim=1, stable=True)[:, :cnt].to(torch.int32)
    return out


def make_inputs(w: Workload, device="cpu", backend="numpy"):
    """Draw the workload's inputs.  Returns a dict of torch tensors on ``device``:
    query, query_rope (dense with rope, else None), key, key_rope, value, dy,
    topk (selected, else None), cu_q, cu_kv (int64, host)."""
    T1, T2 = w.T1, w.T2
    dq_main = w.d_qk
    if backend == "numpy":
        rng = np.random.default_rng([w.seed, 1])
        draw = lambda shape: cast(_normal_np(rng, shape), w.dtype, device)  # noqa: E731
    elif backend == "torch":
        gen = torch.Generator(device=device)
        gen.manual_seed(int(w.seed))
        draw = lambda shape: _normal_torch(gen, shape, device).to(_TORCH_DTYPES[w.dtype])  # noqa: E731
    else:
        raise ValueError(backend)
    out = {}
    out["query"] = draw((T1, w.n1, dq_main))
    out["query_rope"] = draw((T1, w.n1, w.d_rope)) if w.d_rope else None
    out["key"] = draw((T2, w.n2, dq_main))
    out["key_rope"] = draw((T2, w.n2, w.d_rope)) if w.d_rope else None
    out["value"] = draw((T2, w.n2, w.d_v))
    out["dy"] = draw((T1, w.n1, w.d_v))
    out["topk"] = None
    if w.form == "selected":
        cnt = w.block_count
        topk = torch.empty((T1, w.n2, cnt), dtype=torch.int32, device=device)
        cu_q, cu_kv = w.cu_q, w.cu_kv
        for b in range(w.batch):
            qs, qe = int(cu_q[b]), int(cu_q[b + 1])
            nblk = int(cu_kv[b + 1] - cu_kv[b]) // w.block_size
            rows = (qe - qs) * w.n2
            if rows == 0:
                continue
            if backend == "numpy":
                ids = torch.from_numpy(_topk_rows_np(rng, rows, nblk, cnt, w.index_dist, w.zipf_s))
            else:
                ids = _topk_rows_torch(gen, rows, nblk, cnt, w.index_dist, w.zipf_s, device)
            topk[qs:qe] = ids.to(device).reshape(qe - qs, w.n2, cnt)
        out["topk"] = topk
    out["cu_q"] = torch.from_numpy(w.cu_q)
    out["cu_kv"] = torch.from_numpy(w.cu_kv)
    return out


# ----------------------------------------------------------------------------
# lightning-indexer backward inputs
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class IndexerWorkload:
    name: str
    seqlens_q: tuple
    seqlens_kv: tuple
    n1: int
    n2: int
    topk: int
    d: int = 128
    seed: int = 0

    @property
    def batch(self):
        return len(self.seqlens_q)

    @property
    def T1(self):
        return int(sum(self.seqlens_q))

    @property
    def T2(self):
        return int(sum(self.seqlens_kv))

    @property
    def G(self):
        return self.n1 // self.n2

    @property
    def cu_q(self):
        return np.concatenate([[0], np.cumsum(self.seqlens_q)]).astype(np.int64)

    @property
    def cu_kv(self):
        return np.concatenate([[0], np.cumsum(self.seqlens_kv)]).astype(np.int64)


def indexer_config() -> IndexerWorkload:
    """An indexer backward of one 8K sequence: 64 query heads over one key head, D 128, the
    top 2048 keys of each token (seed 6)."""
    return IndexerWorkload("indexer-bf16-S8K-N64-topk2048", (8192,), (8192,), 64, 1, 2048, seed=6)


def small_indexer(seqlens=(96, 64), seqlens_kv=(160, 130), n1=16, n2=1, topk=40, seed=17):
    return IndexerWorkload("indexer-small", tuple(seqlens), tuple(seqlens_kv), n1, n2, topk, seed=seed)


def make_indexer_inputs(w: IndexerWorkload, device="cpu", backend="numpy"):
    """q [T1, N1, D], k [T2, N2, D], weights [T1, N1], dy [T1, N2, topk] ~ N(0, 1) in bf16;
    indices [T1, N2, topk] int32: topk distinct key positions of the token's own sequence,
    uniform (prefix of a random permutation), drawn per (token, key head) in that order."""
    T1, T2 = w.T1, w.T2
    if backend == "numpy":
        rng = np.random.default_rng([w.seed, 2])
        draw = lambda shape: cast(_normal_np(rng, shape), "bf16", device)  # noqa: E731
    else:
        gen = torch.Generator(device=device)
        gen.manual_seed(int(w.seed))
        draw = lambda shape: _normal_torch(gen, shape, device).to(torch.bfloat16)  # noqa: E731
    out = {"q": draw((T1, w.n1, w.d)), "k": draw((T2, w.n2, w.d)), "weights": draw((T1, w.n1)),
           "dy": draw((T1, w.n2, w.topk))}
    idx = torch.empty((T1, w.n2, w.topk), dtype=torch.int32, device=device)
    cu_q, cu_kv = w.cu_q, w.cu_kv
    for b in range(w.batch):
        qs, qe = int(cu_q[b]), int(cu_q[b + 1])
        n = int(cu_kv[b + 1] - cu_kv[b])
        rows = (qe - qs) * w.n2
        if rows == 0:
            continue
        if backend == "numpy":
            ids = torch.from_numpy(_topk_rows_np(rng, rows, n, w.topk, "uniform", 0.0))
        else:
            ids = _topk_rows_torch(gen, rows, n, w.topk, "uniform", 0.0, device)
        idx[qs:qe] = ids.to(device).reshape(qe - qs, w.n2, w.topk)
    out["indices"] = idx
    return out
