"""Float64 CPU oracle for the attention backward pass (dense varlen and NSA selected).

TEST INFRASTRUCTURE ONLY.  This module is imported by the tests, by the smoke
check and by the CPU-baseline leg of the benchmark.  The GPU library never
imports, links or calls it, and it shares no code with the GPU kernels.

What it computes, and where the pages define it
-----------------------------------------------
* Dense form -- page "aclnnFlashAttentionUnpaddingScoreGradV3", Formula section:
  forward  Y = Softmax(Mask(Q K^T / sqrt(d))) V  with  Q = [query, queryRope],
  K = [key, keyRope] concatenated on the head dimension; backward dV = P^T dY,
  dQ = dS K / sqrt(d), dqRope = dS kRope / sqrt(d), dK = dS^T Q / sqrt(d),
  dkRope = dS^T qRope / sqrt(d).  pse and dropout are not used (keep_prob = 1,
  the only value the constraints allow).  Layout is TND (constraints list).
* Selected form -- page "NsaSelectedAttentionGrad" (README), formula section:
  selectedKey / selectedValue are the key / value rows gathered block by block
  through topkIndices (selectedBlockCount blocks of selectedBlockSize rows),
  then the same backward formulas with the printed "V", "Q", "K" read as dV,
  dQ, dK (the outputs are named dqOut/dkOut/dvOut in the parameter table).

Readings taken where the pages are silent (each is listed in the design doc):
* dS is not defined on either page; it is the softmax Jacobian applied to
  dP = dY V^T:  dS = P * (dP - rowsum(P * dP)).
* "1/sqrt(d)" is the caller's scaleValue ("scale") wherever it appears.
* softmaxMax is the row maximum m of the scaled, masked scores and softmaxSum is
  l = sum_j exp(s_j - m); stored as [T, N, 8] float32, 8 identical copies.
* GQA: query head h uses KV head h // G with G = N1 / N2.
* A topk id addresses a block inside its own sequence's KV rows:
  rows cu_kv[b] + id * blockSize + r, r in [0, blockSize).  A repeated id is a
  repeated column (literal Gather); gradients from both copies add up.
* Causal: key j of a sequence is visible to query i of the same sequence when
  j <= i (local positions); it requires equal query and KV lengths.
* The other masks (causal with unequal lengths, windows of preTokens / nextTokens):
  BandMask below; its alignment and window are the reading of sparse modes whose
  definitions the dense page only links to.
* A query row with no visible key produces O = 0 and zero gradients.

The backward recomputes P from the scores (it does not consume the passed
statistics), so it is the exact gradient of <dY, O(Q, K, V)>.  The functions
``backward_*_from_stats`` instead consume the passed O and statistics, the
way the GPU kernels do; they exist to localise a discrepancy.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "BandMask", "forward_dense", "backward_dense", "backward_dense_from_stats",
    "forward_selected", "backward_selected", "backward_selected_from_stats",
    "selected_key_rows", "stats_tensor",
]


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _cat_rope(main, rope):
    """Q = [query, queryRope] (dense page, Formula): concatenate on the head dim."""
    main = _f64(main)
    if rope is None or rope.shape[-1] == 0:
        return main
    return np.concatenate([main, _f64(rope)], axis=-1)


def stats_tensor(m, l):
    """softmaxMax / softmaxSum as the pages shape them: [T, N, 8] float32 copies."""
    m32 = np.asarray(m, dtype=np.float64).astype(np.float32)
    l32 = np.asarray(l, dtype=np.float64).astype(np.float32)
    return (np.repeat(m32[..., None], 8, axis=-1), np.repeat(l32[..., None], 8, axis=-1))


# ----------------------------------------------------------------------------
# Dense varlen form
# ----------------------------------------------------------------------------

class BandMask:
    """A mask on the relative position of key and query (the dense page names sparse modes
    with preTokens / nextTokens and causal variants, but their definitions are not on the
    pages; this is the reading taken).  Key j (position in its sequence) is visible to query i
    when  i + off - pre <= j <= i + off + next,  where off = 0 aligns the first query with the
    first key ("top_left") and off = S2 - S1 aligns the last query with the last key
    ("bottom_right").  pre = inf, next = 0 is causal attention under that alignment."""

    def __init__(self, pre, next, align="top_left"):
        if align not in ("top_left", "bottom_right"):
            raise ValueError(align)
        self.pre, self.next, self.align = pre, next, align

    def visible(self, qpos, n_q, n_k):
        off = 0 if self.align == "top_left" else n_k - n_q
        i = np.asarray(qpos, dtype=np.float64)[:, None]
        j = np.arange(n_k, dtype=np.float64)[None, :]
        return (j >= i + off - self.pre) & (j <= i + off + self.next)


def _causal_mask(qpos, n_q, n_k, causal):
    """Visible[i, j]: the query at local position qpos[i] (of a sequence with n_q
    queries) sees key position j of the same sequence.  causal: False, True (key j
    visible iff j <= i; equal lengths), or a BandMask."""
    if isinstance(causal, BandMask):
        return causal.visible(qpos, n_q, n_k)
    vis = np.ones((len(qpos), n_k), dtype=bool)
    if causal:
        if n_q != n_k:
            raise ValueError("causal attention needs equal query and KV lengths per sequence")
        vis = np.arange(n_k)[None, :] <= np.asarray(qpos)[:, None]
    return vis


def _softmax_rows(S, vis):
    """Row softmax of the masked scores.  Returns P, m, l; a row without any
    visible key gets P = 0, m = -inf, l = 0."""
    Sm = np.where(vis, S, -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, Sm.max(axis=1, initial=-np.inf), -np.inf)
    E = np.where(vis, np.exp(Sm - np.where(any_vis, m, 0.0)[:, None]), 0.0)
    l = E.sum(axis=1)
    P = np.divide(E, l[:, None], out=np.zeros_like(E), where=l[:, None] > 0)
    return P, m, l


def _dense_blocks(cu_q, cu_kv, n1, n2, causal, tokens=None):
    """(query rows, kv slice, visibility mask, query head, KV head) for every
    sequence and query head.  The query rows are the whole sequence, or only the
    listed ``tokens`` that fall in it (ascending)."""
    G = n1 // n2
    toks = None if tokens is None else np.unique(np.asarray(tokens, dtype=np.int64))
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_kv[b]), int(cu_kv[b + 1])
        if toks is None:
            rows = slice(qs, qe)
            qpos = np.arange(qe - qs)
        else:
            rows = toks[(toks >= qs) & (toks < qe)]
            qpos = rows - qs
        if len(qpos) == 0 or ke == ks:
            continue
        vis = _causal_mask(qpos, qe - qs, ke - ks, causal)
        for h in range(n1):
            yield rows, slice(ks, ke), vis, h, h // G


def forward_dense(query, key, value, cu_q, cu_kv, n1, n2, scale, causal,
                  query_rope=None, key_rope=None, tokens=None):
    """Forward of the dense page's Formula section, one (sequence, head) at a time:
    S = Mask(Q K^T * scale), P = Softmax(S), Y = P V.

    Returns O [T1, N1, Dv], m [T1, N1], l [T1, N1] (float64).  Rows without a
    visible key get O = 0, m = -inf, l = 0.  ``tokens`` restricts the work to
    those query tokens (the other rows are left as rows without a visible key).
    """
    Q = _cat_rope(query, query_rope)
    K = _cat_rope(key, key_rope)
    V = _f64(value)
    T1 = Q.shape[0]
    O = np.zeros((T1, n1, V.shape[-1]))
    m = np.full((T1, n1), -np.inf)
    l = np.zeros((T1, n1))
    for qsl, ksl, vis, h, kvh in _dense_blocks(cu_q, cu_kv, n1, n2, causal, tokens):
        S = scale * (Q[qsl, h, :] @ K[ksl, kvh, :].T)
        P, m[qsl, h], l[qsl, h] = _softmax_rows(S, vis)
        O[qsl, h] = P @ V[ksl, kvh, :]
    return O, m, l


def _dense_backward_core(Q, K, V, dY, cu_q, cu_kv, n1, n2, scale, causal, probs_and_D, tokens=None):
    dQ = np.zeros_like(Q)
    dK = np.zeros((K.shape[0], n2, K.shape[-1]))
    dV = np.zeros((V.shape[0], n2, V.shape[-1]))
    for qsl, ksl, vis, h, kvh in _dense_blocks(cu_q, cu_kv, n1, n2, causal, tokens):
        S = scale * (Q[qsl, h, :] @ K[ksl, kvh, :].T)
        dP = dY[qsl, h, :] @ V[ksl, kvh, :].T                    # dP = dY V^T
        P, D = probs_and_D(S, vis, dP, qsl, h)
        dS = P * (dP - D[:, None])                               # softmax Jacobian
        dQ[qsl, h] = scale * (dS @ K[ksl, kvh, :])               # dQ = dS K / sqrt(d)
        dK[ksl, kvh] += scale * (dS.T @ Q[qsl, h, :])            # dK = dS^T Q / sqrt(d)
        dV[ksl, kvh] += P.T @ dY[qsl, h, :]                      # dV = P^T dY
    return dQ, dK, dV


def _split(x, d_main):
    return x[..., :d_main].copy(), x[..., d_main:].copy()


def backward_dense(query, key, value, dy, cu_q, cu_kv, n1, n2, scale, causal,
                   query_rope=None, key_rope=None, tokens=None):
    """Exact gradient for the dense form (P recomputed from the scores).

    Returns dq, dq_rope, dk, dk_rope, dv (float64; the rope parts have 0 columns
    when no rope tensors are given).  With ``tokens`` given, dQ rows of other
    tokens stay 0 and dK / dV hold only the contributions of the listed tokens.
    """
    Q = _cat_rope(query, query_rope)
    K = _cat_rope(key, key_rope)
    V, dY = _f64(value), _f64(dy)

    def exact(S, vis, dP, qsl, h):
        P, _, _ = _softmax_rows(S, vis)
        return P, (P * dP).sum(axis=1)                           # D = sum_j P_j dP_j

    dQ, dK, dV = _dense_backward_core(Q, K, V, dY, cu_q, cu_kv, n1, n2, scale, causal, exact, tokens)
    d_main = np.asarray(query).shape[-1]
    dq, dq_rope = _split(dQ, d_main)
    dk, dk_rope = _split(dK, d_main)
    return dq, dq_rope, dk, dk_rope, dV


def backward_dense_from_stats(query, key, value, out, dy, softmax_max, softmax_sum,
                              cu_q, cu_kv, n1, n2, scale, causal,
                              query_rope=None, key_rope=None, tokens=None):
    """Diagnostic variant consuming the passed statistics and O:
    P = exp(s - m) / l from lane 0 of the stats, D = rowsum(dY * O)."""
    Q = _cat_rope(query, query_rope)
    K = _cat_rope(key, key_rope)
    V, dY, O = _f64(value), _f64(dy), _f64(out)
    m = _f64(softmax_max)[..., 0]
    l = _f64(softmax_sum)[..., 0]

    def consume(S, vis, dP, qsl, h):
        P = np.where(vis, np.exp(np.where(vis, S, 0.0) - m[qsl, h][:, None]), 0.0) / l[qsl, h][:, None]
        return P, (dY[qsl, h] * O[qsl, h]).sum(axis=1)

    dQ, dK, dV = _dense_backward_core(Q, K, V, dY, cu_q, cu_kv, n1, n2, scale, causal, consume, tokens)
    d_main = np.asarray(query).shape[-1]
    dq, dq_rope = _split(dQ, d_main)
    dk, dk_rope = _split(dK, d_main)
    return dq, dq_rope, dk, dk_rope, dV


# ----------------------------------------------------------------------------
# Selected (NSA) form
# ----------------------------------------------------------------------------

def selected_key_rows(ids, kv_start, block_size):
    """Gather(key, topkIndices[i]) for 0 <= i < selectedBlockCount (selected page,
    formula section): the KV rows of the chosen blocks, block after block, in the
    order the ids are given.  Repeated ids repeat their rows."""
    ids = np.asarray(ids, dtype=np.int64)
    return (kv_start + ids[:, None] * block_size + np.arange(block_size)[None, :]).reshape(-1)


def _seq_of_tokens(cu_q, T1):
    seq = np.empty(T1, dtype=np.int64)
    for b in range(len(cu_q) - 1):
        seq[int(cu_q[b]):int(cu_q[b + 1])] = b
    return seq


def _token_list(tokens, T1):
    return range(T1) if tokens is None else [int(t) for t in tokens]


def _scatter_add(dst, rows, vals):
    """ScatterAdd(vals, rows) into dst (selected page; P1's formula names the same
    operation).  A row listed twice receives both contributions."""
    if np.unique(rows).size == rows.size:
        dst[rows] += vals
    else:
        np.add.at(dst, rows, vals)


def forward_selected(query, key, value, topk, cu_q, cu_kv, n1, n2, scale, block_size,
                     tokens=None):
    """Forward of the selected page: for each query token and KV head, attention of
    its G query heads over the gathered selectedKey / selectedValue rows.

    ``tokens`` restricts the work to those query tokens (other rows stay
    O = 0, m = -inf, l = 0).  Returns O [T1, N1, Dv], m, l [T1, N1].
    """
    Q, K, V = _f64(query), _f64(key), _f64(value)
    topk = np.asarray(topk)
    T1 = Q.shape[0]
    G = n1 // n2
    seq = _seq_of_tokens(cu_q, T1)
    O = np.zeros((T1, n1, V.shape[-1]))
    m = np.full((T1, n1), -np.inf)
    l = np.zeros((T1, n1))
    for t in _token_list(tokens, T1):
        ks = int(cu_kv[seq[t]])
        for kvh in range(n2):
            rows = selected_key_rows(topk[t, kvh], ks, block_size)
            heads = slice(kvh * G, (kvh + 1) * G)
            S = scale * (Q[t, heads] @ K[rows, kvh, :].T)          # [G, n]
            P, m[t, heads], l[t, heads] = _softmax_rows(S, np.ones(S.shape, dtype=bool))
            O[t, heads] = P @ V[rows, kvh, :]
    return O, m, l


def _selected_backward_core(Q, K, V, dY, topk, cu_q, cu_kv, n1, n2, scale, block_size,
                            tokens, probs_and_D):
    T1 = Q.shape[0]
    G = n1 // n2
    seq = _seq_of_tokens(cu_q, T1)
    dQ = np.zeros_like(Q)
    # written in full up front: the scatter below first-touches rows in random order,
    # which is far slower than one sequential pass over a large array
    dK = np.full((K.shape[0], n2, K.shape[-1]), 0.0)
    dV = np.full((V.shape[0], n2, V.shape[-1]), 0.0)
    for t in _token_list(tokens, T1):
        ks = int(cu_kv[seq[t]])
        for kvh in range(n2):
            rows = selected_key_rows(topk[t, kvh], ks, block_size)
            heads = slice(kvh * G, (kvh + 1) * G)
            Ks, Vs = K[rows, kvh, :], V[rows, kvh, :]              # selectedKey, selectedValue
            S = scale * (Q[t, heads] @ Ks.T)                        # [G, n]
            dP = dY[t, heads] @ Vs.T                                 # dP = dY V^T
            P, D = probs_and_D(S, dP, t, heads)
            dS = P * (dP - D[:, None])
            dQ[t, heads] = scale * (dS @ Ks)                        # dQ = dS K / sqrt(d)
            _scatter_add(dK[:, kvh, :], rows, scale * (dS.T @ Q[t, heads]))  # dK = dS^T Q / sqrt(d)
            _scatter_add(dV[:, kvh, :], rows, P.T @ dY[t, heads])            # dV = P^T dY
    return dQ, dK, dV


def backward_selected(query, key, value, dy, topk, cu_q, cu_kv, n1, n2, scale, block_size,
                      tokens=None):
    """Exact gradient for the selected form (P recomputed from the scores).

    With ``tokens`` given, dQ rows of other tokens stay 0 and dK / dV hold only
    the contributions of the listed tokens.  Returns dq, dk, dv (float64).
    """
    Q, K, V, dY = _f64(query), _f64(key), _f64(value), _f64(dy)

    def exact(S, dP, t, heads):
        P, _, _ = _softmax_rows(S, np.ones(S.shape, dtype=bool))
        return P, (P * dP).sum(axis=1)

    return _selected_backward_core(Q, K, V, dY, np.asarray(topk), cu_q, cu_kv, n1, n2,
                                   scale, block_size, tokens, exact)


def backward_selected_from_stats(query, key, value, out, dy, softmax_max, softmax_sum, topk,
                                 cu_q, cu_kv, n1, n2, scale, block_size, tokens=None):
    """Diagnostic variant consuming the passed O and statistics (see module doc)."""
    Q, K, V, dY, O = _f64(query), _f64(key), _f64(value), _f64(dy), _f64(out)
    m = _f64(softmax_max)[..., 0]
    l = _f64(softmax_sum)[..., 0]

    def consume(S, dP, t, heads):
        P = np.exp(S - m[t, heads][:, None]) / l[t, heads][:, None]
        return P, (dY[t, heads] * O[t, heads]).sum(axis=1)

    return _selected_backward_core(Q, K, V, dY, np.asarray(topk), cu_q, cu_kv, n1, n2,
                                   scale, block_size, tokens, consume)
