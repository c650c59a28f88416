"""Float64 CPU oracle for the lightning-indexer backward -- TEST INFRASTRUCTURE ONLY.

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg; the GPU
library never imports, links or calls it, and it shares no code with the kernels.

Page "aclnnLightningIndexerGrad", formula section (restated):
    S  = ReLU(Query . Gather(Key, Indices))
    Y  = dy * Weights
    dW = Reduce(S * dy)
    dQ = ReluGrad(Y, S) . Gather(Key, Indices)
    dK = ScatterAdd(ReluGrad(Y, S) . Q, Indices)

The page's parameter table and shape list are lost in its extracted text; the readings
taken (each listed in the design doc):
* Query [T1, N1, D], Key [T2, N2, D] with N1 = G * N2 (the page lists a group G); query
  head h reads key head h // G.
* Indices [T1, N2, topK] int32: for query token t and key head n2, topK key tokens of
  t's own sequence, as positions inside it (the page's S_K constraint "from topK to 128K"
  says a sequence holds at least topK keys).  A repeated index is a repeated column.
* Weights [T1, N1] and dy [T1, N2, topK]: Y[t, h, k] = dy[t, h // G, k] * Weights[t, h], so
  that the scores the backward differentiates are
      out[t, n2, k] = sum_{h in group n2} Weights[t, h] * S[t, h, k],
  and dy is the gradient of out.  No scale factor (the formula has none).
* "Reduce(S * dy)" sums over the selected keys: dW[t, h] = sum_k S[t, h, k] dy[t, h // G, k].
* ReluGrad(Y, S) = Y where S > 0 and 0 elsewhere (the gradient of ReLU at a positive
  pre-activation is 1, at a non-positive one 0).
"""
from __future__ import annotations

import numpy as np

__all__ = ["indexer_forward", "indexer_backward", "indexer_key_rows"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def indexer_key_rows(ids, kv_start):
    """Gather(Key, Indices) for one query token and key head: rows kv_start + id."""
    return kv_start + np.asarray(ids, dtype=np.int64)


def _seq_of_tokens(cu_q, T1):
    seq = np.empty(T1, dtype=np.int64)
    for b in range(len(cu_q) - 1):
        seq[int(cu_q[b]):int(cu_q[b + 1])] = b
    return seq


def indexer_forward(query, key, weights, indices, cu_q, cu_kv, n1, n2):
    """out[t, n2, k] = sum_h Weights[t, h] ReLU(Q[t, h] . K[idx, n2]) over the group's heads.
    Used to pin the backward (finite differences); the page defines only the backward."""
    Q, K, Wt = _f64(query), _f64(key), _f64(weights)
    idx = np.asarray(indices)
    T1, topk = Q.shape[0], idx.shape[-1]
    G = n1 // n2
    seq = _seq_of_tokens(cu_q, T1)
    out = np.zeros((T1, n2, topk))
    for t in range(T1):
        ks = int(cu_kv[seq[t]])
        for kvh in range(n2):
            rows = indexer_key_rows(idx[t, kvh], ks)
            heads = slice(kvh * G, (kvh + 1) * G)
            S = np.maximum(Q[t, heads] @ K[rows, kvh].T, 0.0)          # [G, topK]
            out[t, kvh] = Wt[t, heads] @ S
    return out


def indexer_backward(query, key, weights, dy, indices, cu_q, cu_kv, n1, n2):
    """The page's five formulas, per query token and key head.  Returns dq [T1, N1, D],
    dk [T2, N2, D], dw [T1, N1] (float64)."""
    Q, K, Wt, dY = _f64(query), _f64(key), _f64(weights), _f64(dy)
    idx = np.asarray(indices)
    T1 = Q.shape[0]
    G = n1 // n2
    seq = _seq_of_tokens(cu_q, T1)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dW = np.zeros_like(Wt)
    for t in range(T1):
        ks = int(cu_kv[seq[t]])
        for kvh in range(n2):
            rows = indexer_key_rows(idx[t, kvh], ks)
            heads = slice(kvh * G, (kvh + 1) * G)
            Ks = K[rows, kvh]                                          # Gather(Key, Indices)  [topK, D]
            S = np.maximum(Q[t, heads] @ Ks.T, 0.0)                    # S = ReLU(Q . K)      [G, topK]
            Y = Wt[t, heads][:, None] * dY[t, kvh][None, :]            # Y = dy * Weights
            dW[t, heads] = (S * dY[t, kvh][None, :]).sum(axis=1)       # dW = Reduce(S * dy)
            R = np.where(S > 0.0, Y, 0.0)                              # ReluGrad(Y, S)
            dQ[t, heads] = R @ Ks                                      # dQ = ReluGrad . Gather(K)
            contrib = R.T @ Q[t, heads]                                # [topK, D]
            np.add.at(dK[:, kvh], rows, contrib)                       # dK = ScatterAdd(ReluGrad . Q)
    return dQ, dK, dW
