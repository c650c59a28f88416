"""Pins for the float64 oracle: each test ties it to something other than itself
(finite differences of its own forward, PyTorch autograd of a separately written
naive attention, closed forms derived by hand, exact invariants)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from oracle import attention as OA

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def fd_grad(f, x, h=1e-6):
    """Central finite differences of the scalar f() with respect to array x."""
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        old = x[idx]
        x[idx] = old + h
        fp = f()
        x[idx] = old - h
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


def assert_fd(analytic, fd):
    scale = max(1.0, float(np.abs(fd).max()))
    np.testing.assert_allclose(analytic, fd, rtol=1e-6, atol=1e-7 * scale)


# ----------------------------------------------------------------------------
# finite differences of L = <dY, O(Q, K, V)>
# ----------------------------------------------------------------------------

def _dense_case(rng, lq, lk, n1, n2, d, dr, dv):
    T1, T2 = sum(lq), sum(lk)
    return dict(q=rng.standard_normal((T1, n1, d)), qr=rng.standard_normal((T1, n1, dr)),
                k=rng.standard_normal((T2, n2, d)), kr=rng.standard_normal((T2, n2, dr)),
                v=rng.standard_normal((T2, n2, dv)), dy=rng.standard_normal((T1, n1, dv)))


@pytest.mark.parametrize("causal,lq,lk,n1,n2,dr", [
    (True, (5, 3), (5, 3), 4, 2, 2),          # causal, rope split, GQA G=2
    (False, (4, 0, 3), (2, 3, 5), 2, 1, 0),   # unequal lengths, empty query sequence, G=2
    (True, (6,), (6,), 4, 1, 3),              # G=4
])
def test_dense_backward_matches_finite_differences(causal, lq, lk, n1, n2, dr):
    rng = np.random.default_rng(7)
    c = _dense_case(rng, lq, lk, n1, n2, 6, dr, 5)
    cq, ck, scale = cu(lq), cu(lk), 0.37

    def loss():
        o, _, _ = O.forward_dense(c["q"], c["k"], c["v"], cq, ck, n1, n2, scale, causal, c["qr"], c["kr"])
        return float((c["dy"] * o).sum())

    dq, dqr, dk, dkr, dv = O.backward_dense(c["q"], c["k"], c["v"], c["dy"], cq, ck, n1, n2, scale,
                                            causal, c["qr"], c["kr"])
    assert_fd(dq, fd_grad(loss, c["q"]))
    assert_fd(dk, fd_grad(loss, c["k"]))
    assert_fd(dv, fd_grad(loss, c["v"]))
    if dr:
        assert_fd(dqr, fd_grad(loss, c["qr"]))
        assert_fd(dkr, fd_grad(loss, c["kr"]))


def _selected_case(rng, lq, lk, n1, n2, d, dv, bs, cnt, dup=False):
    T1, T2 = sum(lq), sum(lk)
    topk = np.zeros((T1, n2, cnt), dtype=np.int32)
    cq = cu(lq)
    for b in range(len(lq)):
        nblk = lk[b] // bs
        for t in range(cq[b], cq[b + 1]):
            for h in range(n2):
                topk[t, h] = rng.permutation(nblk)[:cnt]
                if dup and (t + h) % 3 == 0:
                    topk[t, h, -1] = topk[t, h, 0]     # a repeated id
    return dict(q=rng.standard_normal((T1, n1, d)), k=rng.standard_normal((T2, n2, d)),
                v=rng.standard_normal((T2, n2, dv)), dy=rng.standard_normal((T1, n1, dv)), topk=topk)


@pytest.mark.parametrize("dup", [False, True])
def test_selected_backward_matches_finite_differences(dup):
    rng = np.random.default_rng(8)
    lq, lk, n1, n2, bs, cnt = (4, 3), (6, 8), 4, 2, 2, 3
    c = _selected_case(rng, lq, lk, n1, n2, 5, 4, bs, cnt, dup)
    cq, ck, scale = cu(lq), cu(lk), 0.41

    def loss():
        o, _, _ = O.forward_selected(c["q"], c["k"], c["v"], c["topk"], cq, ck, n1, n2, scale, bs)
        return float((c["dy"] * o).sum())

    dq, dk, dv = O.backward_selected(c["q"], c["k"], c["v"], c["dy"], c["topk"], cq, ck, n1, n2, scale, bs)
    assert_fd(dq, fd_grad(loss, c["q"]))
    assert_fd(dk, fd_grad(loss, c["k"]))
    assert_fd(dv, fd_grad(loss, c["v"]))


def test_finite_differences_catch_a_dropped_jacobian_term():
    """A planted mistake in the oracle (dS = P * dP, the rowsum term dropped) must
    fail the finite-difference pin."""
    rng = np.random.default_rng(9)
    lq, n1, n2 = (5,), 2, 1
    c = _dense_case(rng, lq, lq, n1, n2, 4, 0, 3)
    cq = cu(lq)

    def wrong(S, vis, dP, qsl, h):
        P, _, _ = OA._softmax_rows(S, vis)
        return P, np.zeros(P.shape[0])

    dq_bad, _, _ = OA._dense_backward_core(c["q"], c["k"], c["v"], c["dy"], cq, cq, n1, n2, 0.5, True, wrong)

    def loss():
        o, _, _ = O.forward_dense(c["q"], c["k"], c["v"], cq, cq, n1, n2, 0.5, True)
        return float((c["dy"] * o).sum())

    with pytest.raises(AssertionError):
        assert_fd(dq_bad, fd_grad(loss, c["q"]))


# ----------------------------------------------------------------------------
# PyTorch float64 autograd of a separately written naive attention
# ----------------------------------------------------------------------------

def _torch_dense_loss(q, qr, k, kr, v, dy, lq, lk, n1, n2, scale, causal):
    G = n1 // n2
    total = q.new_zeros(())
    cq, ck = cu(lq), cu(lk)
    for b in range(len(lq)):
        if lq[b] == 0 or lk[b] == 0:
            continue
        Qb = torch.cat([q[cq[b]:cq[b + 1]], qr[cq[b]:cq[b + 1]]], -1).transpose(0, 1)     # [N1, Sq, D]
        Kb = torch.cat([k[ck[b]:ck[b + 1]], kr[ck[b]:ck[b + 1]]], -1).transpose(0, 1)
        Vb = v[ck[b]:ck[b + 1]].transpose(0, 1)
        Kb, Vb = Kb.repeat_interleave(G, 0), Vb.repeat_interleave(G, 0)                 # [N1, Sk, D]
        S = torch.matmul(Qb, Kb.transpose(1, 2).contiguous()) * scale
        if causal:
            mask = torch.ones(lq[b], lk[b], dtype=torch.bool).triu(1)
            S = S.masked_fill(mask, float("-inf"))
        Ob = torch.matmul(torch.softmax(S, -1), Vb).transpose(0, 1)
        total = total + (dy[cq[b]:cq[b + 1]] * Ob).sum()
    return total


def test_dense_backward_matches_torch_autograd():
    rng = np.random.default_rng(10)
    lq = (33, 17)
    n1, n2, scale = 4, 2, 0.29
    c = _dense_case(rng, lq, lq, n1, n2, 16, 8, 12)
    ts = {k: torch.tensor(v, requires_grad=True) for k, v in c.items()}
    _torch_dense_loss(ts["q"], ts["qr"], ts["k"], ts["kr"], ts["v"], ts["dy"], lq, lq, n1, n2, scale,
                      True).backward()
    got = O.backward_dense(c["q"], c["k"], c["v"], c["dy"], cu(lq), cu(lq), n1, n2, scale, True,
                           c["qr"], c["kr"])
    for mine, name in zip(got, ["q", "qr", "k", "kr", "v"]):
        np.testing.assert_allclose(mine, ts[name].grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("dup", [False, True])
def test_selected_backward_matches_torch_autograd(dup):
    rng = np.random.default_rng(12)
    lq, lk, n1, n2, bs, cnt = (20, 12), (32, 48), 8, 2, 4, 5
    c = _selected_case(rng, lq, lk, n1, n2, 12, 8, bs, cnt, dup)
    cq, ck, scale = cu(lq), cu(lk), 0.33
    G = n1 // n2
    q, k, v = (torch.tensor(c[x], requires_grad=True) for x in ("q", "k", "v"))
    dy = torch.tensor(c["dy"])
    # row indices of the gathered keys, [T1, N2, cnt*bs], built with torch ops
    seq = torch.repeat_interleave(torch.arange(len(lq)), torch.tensor(lq))
    ids = torch.tensor(c["topk"]).long()
    rows = (torch.tensor(ck)[seq][:, None, None, None] + ids[..., None] * bs
            + torch.arange(bs)[None, None, None, :]).reshape(sum(lq), n2, cnt * bs)
    kv_head = torch.arange(n2)[None, :, None].expand_as(rows)
    Ks, Vs = k[rows, kv_head], v[rows, kv_head]                     # [T1, N2, n, D]
    Qg = q.reshape(sum(lq), n2, G, -1)
    S = torch.matmul(Qg, Ks.transpose(-1, -2).contiguous()) * scale  # [T1, N2, G, n]
    Og = torch.matmul(torch.softmax(S, -1), Vs)
    (dy.reshape(sum(lq), n2, G, -1) * Og).sum().backward()
    dq, dk, dv = O.backward_selected(c["q"], c["k"], c["v"], c["dy"], c["topk"], cq, ck, n1, n2, scale, bs)
    np.testing.assert_allclose(dq, q.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, k.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, v.grad.numpy(), rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------
# selected <-> dense, invariants, closed forms
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("order", ["identity", "reversed"])
def test_selected_with_every_block_equals_dense_noncausal(order):
    rng = np.random.default_rng(14)
    lens, n1, n2, bs, cnt, scale = (24, 24), 4, 2, 8, 3, 0.3
    c = _dense_case(rng, lens, lens, n1, n2, 10, 0, 6)
    ids = np.arange(cnt) if order == "identity" else np.arange(cnt)[::-1]
    topk = np.broadcast_to(ids, (sum(lens), n2, cnt)).astype(np.int32)
    dq_s, dk_s, dv_s = O.backward_selected(c["q"], c["k"], c["v"], c["dy"], topk, cu(lens), cu(lens),
                                           n1, n2, scale, bs)
    dq_d, _, dk_d, _, dv_d = O.backward_dense(c["q"], c["k"], c["v"], c["dy"], cu(lens), cu(lens),
                                              n1, n2, scale, False)
    for a, b in ((dq_s, dq_d), (dk_s, dk_d), (dv_s, dv_d)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    o_s, m_s, l_s = O.forward_selected(c["q"], c["k"], c["v"], topk, cu(lens), cu(lens), n1, n2, scale, bs)
    o_d, m_d, l_d = O.forward_dense(c["q"], c["k"], c["v"], cu(lens), cu(lens), n1, n2, scale, False)
    np.testing.assert_allclose(o_s, o_d, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(m_s, m_d, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l_s, l_d, rtol=1e-12, atol=1e-12)


def _group_sums(x, cuk, n2):
    return np.stack([x[cuk[b]:cuk[b + 1]].sum(axis=0) for b in range(len(cuk) - 1)])


def test_gradient_invariants_dense():
    """rowsum(dS) = 0 gives sum_j dK_j = 0 per (sequence, KV head); rows of P sum to 1
    gives sum_j dV_j = sum of dY over the group's query rows; dQ is unchanged when a
    constant vector is added to every key of a (sequence, KV head)."""
    rng = np.random.default_rng(15)
    lens, n1, n2, scale = (9, 14), 6, 2, 0.35
    c = _dense_case(rng, lens, lens, n1, n2, 8, 4, 5)
    cl = cu(lens)
    dq, dqr, dk, dkr, dv = O.backward_dense(c["q"], c["k"], c["v"], c["dy"], cl, cl, n1, n2, scale, True,
                                            c["qr"], c["kr"])
    assert np.abs(_group_sums(dk, cl, n2)).max() < 1e-12
    assert np.abs(_group_sums(dkr, cl, n2)).max() < 1e-12
    G = n1 // n2
    dy_groups = c["dy"].reshape(-1, n2, G, c["dy"].shape[-1]).sum(axis=2)
    np.testing.assert_allclose(_group_sums(dv, cl, n2), _group_sums(dy_groups, cl, n2), atol=1e-12)
    shift = rng.standard_normal((len(lens), n2, 8))
    k2 = c["k"].copy()
    for b in range(len(lens)):
        k2[cl[b]:cl[b + 1]] += shift[b][None]
    dq2, dqr2, _, _, _ = O.backward_dense(c["q"], k2, c["v"], c["dy"], cl, cl, n1, n2, scale, True,
                                          c["qr"], c["kr"])
    np.testing.assert_allclose(dq2 - dq, np.zeros_like(dq), atol=1e-9)


def test_gradient_invariants_selected():
    rng = np.random.default_rng(16)
    lq, lk, n1, n2, bs, cnt = (10, 7), (16, 24), 4, 2, 4, 3
    c = _selected_case(rng, lq, lk, n1, n2, 6, 5, bs, cnt, dup=True)
    cq, ck, scale = cu(lq), cu(lk), 0.5
    dq, dk, dv = O.backward_selected(c["q"], c["k"], c["v"], c["dy"], c["topk"], cq, ck, n1, n2, scale, bs)
    assert np.abs(_group_sums(dk, ck, n2)).max() < 1e-12
    G = n1 // n2
    dy_groups = c["dy"].reshape(-1, n2, G, c["dy"].shape[-1]).sum(axis=2)
    np.testing.assert_allclose(_group_sums(dv, ck, n2), _group_sums(dy_groups, cq, n2), atol=1e-12)


def test_zero_queries_closed_form():
    """Q = 0 makes every score 0, so P = 1/n on each row.  By hand from the forward:
    dV_j = (1/n) sum_rows dY, dK = 0, and
    dQ = scale * (1/n) * sum_j K_j * ((V_j - mean V) . dY)."""
    rng = np.random.default_rng(17)
    n, n1, n2, scale = 7, 2, 1, 0.6
    c = _dense_case(rng, (n,), (n,), n1, n2, 4, 0, 3)
    q = np.zeros_like(c["q"])
    dq, _, dk, _, dv = O.backward_dense(q, c["k"], c["v"], c["dy"], cu((n,)), cu((n,)), n1, n2, scale, False)
    K, V, dY = c["k"][:, 0], c["v"][:, 0], c["dy"]
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv[:, 0], np.broadcast_to(dY.sum(axis=(0, 1)) / n, V.shape), atol=1e-14)
    Vc = V - V.mean(axis=0)
    for t in range(n):
        for h in range(n1):
            want = scale / n * sum(K[j] * (Vc[j] @ dY[t, h]) for j in range(n))
            np.testing.assert_allclose(dq[t, h], want, atol=1e-14)


def test_single_key_closed_form():
    """One visible key: P = 1 and dS = 0, so dQ = dK = 0 and dV = sum of dY."""
    rng = np.random.default_rng(18)
    c = _dense_case(rng, (1, 3), (1, 1), 2, 1, 4, 2, 3)
    dq, dqr, dk, dkr, dv = O.backward_dense(c["q"], c["k"], c["v"], c["dy"], cu((1, 3)), cu((1, 1)), 2, 1,
                                            0.5, False, c["qr"], c["kr"])
    for x in (dq, dqr, dk, dkr):
        np.testing.assert_allclose(x, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv[0, 0], c["dy"][0:1].sum(axis=(0, 1)), atol=1e-14)
    np.testing.assert_allclose(dv[1, 0], c["dy"][1:4].sum(axis=(0, 1)), atol=1e-14)


def test_golden_two_key_hand_derivation():
    g = json.load(open(os.path.join(GOLDEN, "two_key_uniform.json")))
    i, e = g["inputs"], g["expected"]
    q = np.array(i["q"]).reshape(1, 1, 1)
    k = np.array(i["k"]).reshape(2, 1, 1)
    v = np.array(i["v"]).reshape(2, 1, 1)
    dy = np.array(i["dy"]).reshape(1, 1, 1)
    cq, ck = cu((1,)), cu((2,))
    o, m, l = O.forward_dense(q, k, v, cq, ck, 1, 1, i["scale"], False)
    dq, _, dk, _, dv = O.backward_dense(q, k, v, dy, cq, ck, 1, 1, i["scale"], False)
    assert o.ravel().tolist() == pytest.approx(e["o"], abs=1e-15)
    assert dq.ravel().tolist() == pytest.approx(e["dq"], abs=1e-15)
    assert dk.ravel().tolist() == pytest.approx(e["dk"], abs=1e-15)
    assert dv.ravel().tolist() == pytest.approx(e["dv"], abs=1e-15)
    assert float(m[0, 0]) == pytest.approx(e["m"]) and float(l[0, 0]) == pytest.approx(e["l"])


def test_logistic_two_key_closed_form():
    """Two keys: O = s(x) v1 + (1 - s(x)) v2 with x = scale q.(k1 - k2) and s the logistic
    function; the gradient follows by hand from s' = s (1 - s)."""
    rng = np.random.default_rng(19)
    d, dvd, scale = 5, 3, 0.7
    q, k, v, dy = (rng.standard_normal(s) for s in ((1, 1, d), (2, 1, d), (2, 1, dvd), (1, 1, dvd)))
    dq, _, dk, _, dv = O.backward_dense(q, k, v, dy, cu((1,)), cu((2,)), 1, 1, scale, False)
    k1, k2, v1, v2, qq, g = k[0, 0], k[1, 0], v[0, 0], v[1, 0], q[0, 0], dy[0, 0]
    x = scale * qq @ (k1 - k2)
    s = 1.0 / (1.0 + math.exp(-x))
    ds = s * (1 - s) * (g @ (v1 - v2))
    np.testing.assert_allclose(dq[0, 0], scale * ds * (k1 - k2), atol=1e-14)
    np.testing.assert_allclose(dk[0, 0], scale * ds * qq, atol=1e-14)
    np.testing.assert_allclose(dk[1, 0], -scale * ds * qq, atol=1e-14)
    np.testing.assert_allclose(dv[0, 0], s * g, atol=1e-14)
    np.testing.assert_allclose(dv[1, 0], (1 - s) * g, atol=1e-14)


# ----------------------------------------------------------------------------
# statistics: the forward's (m, l) and O reproduce the exact gradient
# ----------------------------------------------------------------------------

def test_stats_semantics_dense():
    """Consuming float64 (m, l) and O from the forward reproduces the exact gradient,
    which fixes m as the row max of the scaled masked scores and l as sum exp(s - m)."""
    rng = np.random.default_rng(20)
    lens, n1, n2, scale = (12, 5), 4, 2, 0.4
    c = _dense_case(rng, lens, lens, n1, n2, 6, 2, 4)
    cl = cu(lens)
    o, m, l = O.forward_dense(c["q"], c["k"], c["v"], cl, cl, n1, n2, scale, True, c["qr"], c["kr"])
    m8, l8 = np.repeat(m[..., None], 8, -1), np.repeat(l[..., None], 8, -1)
    a = O.backward_dense(c["q"], c["k"], c["v"], c["dy"], cl, cl, n1, n2, scale, True, c["qr"], c["kr"])
    b = O.backward_dense_from_stats(c["q"], c["k"], c["v"], o, c["dy"], m8, l8, cl, cl, n1, n2, scale, True,
                                    c["qr"], c["kr"])
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)
    # row max of the scores is attained: the largest exp(s - m) is exactly 1 (P_max = 1/l)
    S = scale * (np.concatenate([c["q"], c["qr"]], -1)[:12, 0] @ np.concatenate([c["k"], c["kr"]], -1)[:12, 0].T)
    S = np.where(np.tril(np.ones((12, 12), bool)), S, -np.inf)
    np.testing.assert_allclose(S.max(axis=1), m[:12, 0], rtol=1e-14)


def test_stats_semantics_selected():
    rng = np.random.default_rng(21)
    lq, lk, n1, n2, bs, cnt = (6, 5), (8, 12), 4, 2, 2, 3
    c = _selected_case(rng, lq, lk, n1, n2, 5, 4, bs, cnt, dup=True)
    cq, ck, scale = cu(lq), cu(lk), 0.45
    o, m, l = O.forward_selected(c["q"], c["k"], c["v"], c["topk"], cq, ck, n1, n2, scale, bs)
    m8, l8 = np.repeat(m[..., None], 8, -1), np.repeat(l[..., None], 8, -1)
    a = O.backward_selected(c["q"], c["k"], c["v"], c["dy"], c["topk"], cq, ck, n1, n2, scale, bs)
    b = O.backward_selected_from_stats(c["q"], c["k"], c["v"], o, c["dy"], m8, l8, c["topk"], cq, ck, n1, n2,
                                       scale, bs)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)


def test_stats_tensor_layout():
    m = np.array([[1.0, 2.0]])
    l = np.array([[3.0, 4.0]])
    m8, l8 = O.stats_tensor(m, l)
    assert m8.shape == (1, 2, 8) and m8.dtype == np.float32
    assert (m8 == np.array([1.0, 2.0], np.float32)[None, :, None]).all()
    assert (l8[0, 1] == 4.0).all()


def test_token_subset_matches_full_run():
    """The sampled-token mode used at full sizes equals the full run on those tokens."""
    rng = np.random.default_rng(22)
    lq, lk, n1, n2, bs, cnt = (6, 5), (8, 12), 4, 2, 2, 3
    c = _selected_case(rng, lq, lk, n1, n2, 5, 4, bs, cnt)
    cq, ck, scale = cu(lq), cu(lk), 0.45
    full = O.backward_selected(c["q"], c["k"], c["v"], c["dy"], c["topk"], cq, ck, n1, n2, scale, bs)
    toks = [1, 7]
    part = O.backward_selected(c["q"], c["k"], c["v"], c["dy"], c["topk"], cq, ck, n1, n2, scale, bs,
                               tokens=toks)
    np.testing.assert_allclose(part[0][toks], full[0][toks], rtol=1e-13)
    # a key row selected only by the listed tokens has the full gradient
    only = O.backward_selected(c["q"], c["k"], c["v"], c["dy"], c["topk"], cq, ck, n1, n2, scale, bs,
                               tokens=range(sum(lq)))
    np.testing.assert_allclose(only[1], full[1], rtol=1e-13)


def _inert_stats(m, l, o, tokens):
    """Statistics and O for rows outside ``tokens`` that make those rows contribute
    nothing: l = 1 and a maximum far above every score give P = exp(s - m) / l = 0,
    and O = 0 gives rowsum(dY * O) = 0, hence dS = 0."""
    keep = np.zeros(m.shape[0], dtype=bool)
    keep[list(tokens)] = True
    m, l, o = m.copy(), l.copy(), o.copy()
    m[~keep] = 3.0e4
    l[~keep] = 1.0
    o[~keep] = 0.0
    return m, l, o


def test_dense_token_subset_is_additive():
    """Rows of disjoint token subsets: forward rows and dQ rows equal the full run's,
    and the dK / dV contributions of the two subsets add up to the full gradient."""
    rng = np.random.default_rng(23)
    lq, n1, n2, dr = (7, 0, 9), 4, 2, 3
    c = _dense_case(rng, lq, lq, n1, n2, 6, dr, 5)
    cq, scale = cu(lq), 0.41
    args = (cq, cq, n1, n2, scale, True)
    fo, fm, fl = O.forward_dense(c["q"], c["k"], c["v"], *args, c["qr"], c["kr"])
    full = O.backward_dense(c["q"], c["k"], c["v"], c["dy"], *args, c["qr"], c["kr"])
    A = [0, 3, 6, 8, 15]
    B = sorted(set(range(sum(lq))) - set(A))
    po, pm, pl = O.forward_dense(c["q"], c["k"], c["v"], *args, c["qr"], c["kr"], tokens=A)
    np.testing.assert_allclose(po[A], fo[A], rtol=1e-13)
    np.testing.assert_allclose(pm[A], fm[A], rtol=1e-13)
    assert np.isneginf(pm[B]).all() and (pl[B] == 0).all() and (po[B] == 0).all()
    ga = O.backward_dense(c["q"], c["k"], c["v"], c["dy"], *args, c["qr"], c["kr"], tokens=A)
    gb = O.backward_dense(c["q"], c["k"], c["v"], c["dy"], *args, c["qr"], c["kr"], tokens=B)
    for i in (0, 1):   # dq, dq_rope: row restriction
        np.testing.assert_allclose(ga[i][A], full[i][A], rtol=1e-12, atol=1e-14)
        assert (ga[i][B] == 0).all()
    for i in (2, 3, 4):  # dk, dk_rope, dv: additivity over query rows
        np.testing.assert_allclose(ga[i] + gb[i], full[i], rtol=1e-12, atol=1e-13)


def test_inert_rows_contribute_nothing_dense():
    """The construction of the full-size parity tests: rows outside the sampled tokens
    get O = 0, l = 1 and a huge maximum; consuming those statistics the way the kernels
    do gives exactly the gradient of the sampled rows alone."""
    rng = np.random.default_rng(24)
    lq, n1, n2, dr = (8, 6), 4, 2, 2
    c = _dense_case(rng, lq, lq, n1, n2, 6, dr, 5)
    cq, scale = cu(lq), 0.39
    args = (cq, cq, n1, n2, scale, True)
    toks = [1, 5, 9, 13]
    o, m, l = O.forward_dense(c["q"], c["k"], c["v"], *args, c["qr"], c["kr"], tokens=toks)
    m, l, o = _inert_stats(m, l, o, toks)
    smax, ssum = m[..., None].repeat(8, -1), l[..., None].repeat(8, -1)
    got = O.backward_dense_from_stats(c["q"], c["k"], c["v"], o, c["dy"], smax, ssum, *args, c["qr"], c["kr"])
    want = O.backward_dense(c["q"], c["k"], c["v"], c["dy"], *args, c["qr"], c["kr"], tokens=toks)
    for g, wv in zip(got, want):
        np.testing.assert_allclose(g, wv, rtol=1e-10, atol=1e-12)


def test_inert_rows_contribute_nothing_selected():
    rng = np.random.default_rng(25)
    lq, lk, n1, n2, bs, cnt = (6, 5), (8, 12), 4, 2, 2, 3
    c = _selected_case(rng, lq, lk, n1, n2, 5, 4, bs, cnt)
    cq, ck, scale = cu(lq), cu(lk), 0.45
    args = (c["topk"], cq, ck, n1, n2, scale, bs)
    toks = [0, 4, 7]
    o, m, l = O.forward_selected(c["q"], c["k"], c["v"], *args, tokens=toks)
    m, l, o = _inert_stats(m, l, o, toks)
    smax, ssum = m[..., None].repeat(8, -1), l[..., None].repeat(8, -1)
    got = O.backward_selected_from_stats(c["q"], c["k"], c["v"], o, c["dy"], smax, ssum, *args)
    want = O.backward_selected(c["q"], c["k"], c["v"], c["dy"], *args, tokens=toks)
    for g, wv in zip(got, want):
        np.testing.assert_allclose(g, wv, rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------
# band / alignment masks (BandMask): causal with unequal lengths, preTokens / nextTokens
# ----------------------------------------------------------------------------

INF = float("inf")
BANDS = [
    ("causal-bottom-right, S1 < S2", (4, 3), (7, 5), OA.BandMask(INF, 0, "bottom_right")),
    ("causal-bottom-right, S1 > S2 (rows with no key)", (6, 2), (3, 2), OA.BandMask(INF, 0, "bottom_right")),
    ("causal-top-left, S1 < S2", (4, 3), (7, 5), OA.BandMask(INF, 0, "top_left")),
    ("band pre 2 next 1, bottom-right", (5, 4), (6, 4), OA.BandMask(2, 1, "bottom_right")),
    ("band pre 0 next 3, top-left", (5,), (5,), OA.BandMask(0, 3, "top_left")),
]


@pytest.mark.parametrize("name,lq,lk,mask", BANDS, ids=[b[0] for b in BANDS])
def test_band_mask_backward_matches_finite_differences(name, lq, lk, mask):
    rng = np.random.default_rng(21)
    n1, n2, dr = 4, 2, 2
    c = _dense_case(rng, lq, lk, n1, n2, 5, dr, 4)
    cq, ck, scale = cu(lq), cu(lk), 0.43

    def loss():
        o, _, _ = O.forward_dense(c["q"], c["k"], c["v"], cq, ck, n1, n2, scale, mask, c["qr"], c["kr"])
        return float((c["dy"] * o).sum())

    dq, dqr, dk, dkr, dv = O.backward_dense(c["q"], c["k"], c["v"], c["dy"], cq, ck, n1, n2, scale, mask,
                                            c["qr"], c["kr"])
    assert_fd(dq, fd_grad(loss, c["q"]))
    assert_fd(dk, fd_grad(loss, c["k"]))
    assert_fd(dv, fd_grad(loss, c["v"]))
    assert_fd(dkr, fd_grad(loss, c["kr"]))


def _torch_band_loss(q, k, v, dy, lq, lk, n1, n2, scale, lo_rel, hi_rel, bottom_right):
    """Naive attention with the mask built by torch.tril / triu diagonals (independent of BandMask):
    visible iff lo <= j - i <= hi with lo, hi shifted by S2 - S1 when aligned bottom-right."""
    G = n1 // n2
    total = q.new_zeros(())
    cq, ck = cu(lq), cu(lk)
    for b in range(len(lq)):
        s1, s2 = lq[b], lk[b]
        off = s2 - s1 if bottom_right else 0
        keep = torch.ones(s1, s2, dtype=torch.bool).tril(off + hi_rel) & torch.ones(s1, s2, dtype=torch.bool).triu(
            off + lo_rel)
        Qb = q[cq[b]:cq[b + 1]].transpose(0, 1)
        Kb = k[ck[b]:ck[b + 1]].transpose(0, 1).repeat_interleave(G, 0)
        Vb = v[ck[b]:ck[b + 1]].transpose(0, 1).repeat_interleave(G, 0)
        S = torch.matmul(Qb, Kb.transpose(1, 2).contiguous()) * scale
        S = S.masked_fill(~keep, float("-inf"))
        P = torch.softmax(S, -1).nan_to_num(0.0)   # a row with no visible key: P = 0
        total = total + (dy[cq[b]:cq[b + 1]] * torch.matmul(P, Vb).transpose(0, 1)).sum()
    return total


@pytest.mark.parametrize("lo_rel,hi_rel,bottom_right,lq,lk", [
    (-1000, 0, True, (9, 5), (13, 5)),
    (-1000, 0, True, (8,), (5,)),
    (-3, 2, True, (7, 6), (9, 6)),
    (-2, 4, False, (7,), (10,)),
])
def test_band_mask_matches_torch_autograd(lo_rel, hi_rel, bottom_right, lq, lk):
    rng = np.random.default_rng(22)
    n1, n2, scale = 4, 2, 0.31
    c = _dense_case(rng, lq, lk, n1, n2, 8, 0, 6)
    ts = {k: torch.tensor(v, requires_grad=True) for k, v in c.items()}
    _torch_band_loss(ts["q"], ts["k"], ts["v"], ts["dy"], lq, lk, n1, n2, scale, lo_rel, hi_rel,
                     bottom_right).backward()
    mask = OA.BandMask(-lo_rel, hi_rel, "bottom_right" if bottom_right else "top_left")
    dq, _, dk, _, dv = O.backward_dense(c["q"], c["k"], c["v"], c["dy"], cu(lq), cu(lk), n1, n2, scale, mask)
    for mine, name in zip((dq, dk, dv), ("q", "k", "v")):
        np.testing.assert_allclose(mine, ts[name].grad.numpy(), rtol=1e-11, atol=1e-12)


def test_band_mask_special_cases():
    """Equal lengths: both alignments of causal are the causal mask; a window wider than the
    sequences is no mask; a bottom-right causal row before the first key has no key at all."""
    rng = np.random.default_rng(23)
    lq = (6, 4)
    c = _dense_case(rng, lq, lq, 2, 1, 4, 0, 3)
    ref = O.forward_dense(c["q"], c["k"], c["v"], cu(lq), cu(lq), 2, 1, 0.5, True)
    for align in ("top_left", "bottom_right"):
        got = O.forward_dense(c["q"], c["k"], c["v"], cu(lq), cu(lq), 2, 1, 0.5, OA.BandMask(INF, 0, align))
        for a, b in zip(got, ref):
            np.testing.assert_array_equal(a, b)
    full = O.forward_dense(c["q"], c["k"], c["v"], cu(lq), cu(lq), 2, 1, 0.5, False)
    wide = O.forward_dense(c["q"], c["k"], c["v"], cu(lq), cu(lq), 2, 1, 0.5, OA.BandMask(100, 100))
    for a, b in zip(wide, full):
        np.testing.assert_array_equal(a, b)
    o, m, l = O.forward_dense(c["q"][:6], c["k"][:4], c["v"][:4], cu((6,)), cu((4,)), 2, 1, 0.5,
                              OA.BandMask(INF, 0, "bottom_right"))
    assert (o[:2] == 0).all() and np.isneginf(m[:2]).all() and (l[:2] == 0).all()   # rows 0, 1: no key
    assert (l[2:] > 0).all()
