"""Pins for the lightning-indexer oracle (oracle/indexer.py): finite differences of its own
forward, PyTorch float64 autograd of a separately written forward, a planted mistake, and
closed forms."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import indexer as OI


def cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def case(rng, lq, lk, n1, n2, d, topk, dup=False):
    T1, T2 = sum(lq), sum(lk)
    idx = np.zeros((T1, n2, topk), dtype=np.int32)
    cq = cu(lq)
    for b in range(len(lq)):
        for t in range(cq[b], cq[b + 1]):
            for h in range(n2):
                idx[t, h] = rng.permutation(lk[b])[:topk]
                if dup and (t + h) % 2 == 0:
                    idx[t, h, -1] = idx[t, h, 0]
    return dict(q=rng.standard_normal((T1, n1, d)), k=rng.standard_normal((T2, n2, d)),
                w=rng.standard_normal((T1, n1)), dy=rng.standard_normal((T1, n2, topk)), idx=idx)


def fd_grad(f, x, h=1e-6):
    g = np.zeros_like(x)
    for i in np.ndindex(x.shape):
        old = x[i]
        x[i] = old + h
        fp = f()
        x[i] = old - h
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


def assert_fd(a, b):
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-7 * max(1.0, float(np.abs(b).max())))


@pytest.mark.parametrize("dup", [False, True])
def test_indexer_backward_matches_finite_differences(dup):
    rng = np.random.default_rng(31)
    lq, lk, n1, n2, d, topk = (3, 2), (6, 5), 4, 2, 5, 4
    c = case(rng, lq, lk, n1, n2, d, topk, dup)
    cq, ck = cu(lq), cu(lk)

    def loss():
        return float((c["dy"] * O.indexer_forward(c["q"], c["k"], c["w"], c["idx"], cq, ck, n1, n2)).sum())

    dq, dk, dw = O.indexer_backward(c["q"], c["k"], c["w"], c["dy"], c["idx"], cq, ck, n1, n2)
    assert_fd(dq, fd_grad(loss, c["q"]))
    assert_fd(dk, fd_grad(loss, c["k"]))
    assert_fd(dw, fd_grad(loss, c["w"]))


def test_indexer_planted_mistake_fails_the_pin():
    """Without the ReLU gradient mask (ReluGrad(Y, S) = Y everywhere) the pin must fail."""
    rng = np.random.default_rng(32)
    lq, lk, n1, n2, d, topk = (3,), (6,), 2, 1, 4, 4
    c = case(rng, lq, lk, n1, n2, d, topk)
    cq, ck = cu(lq), cu(lk)
    G = n1 // n2
    Q, K = c["q"], c["k"]
    dq_bad = np.zeros_like(Q)
    for t in range(3):
        Ks = K[c["idx"][t, 0], 0]
        Y = c["w"][t][:, None] * c["dy"][t, 0][None, :]
        dq_bad[t] = Y @ Ks                                            # the mask dropped

    def loss():
        return float((c["dy"] * O.indexer_forward(Q, K, c["w"], c["idx"], cq, ck, n1, n2)).sum())

    with pytest.raises(AssertionError):
        assert_fd(dq_bad, fd_grad(loss, Q))
    assert G == 2


def test_indexer_backward_matches_torch_autograd():
    rng = np.random.default_rng(33)
    lq, lk, n1, n2, d, topk = (7, 5), (12, 9), 8, 2, 16, 6
    c = case(rng, lq, lk, n1, n2, d, topk, dup=True)
    cq, ck = cu(lq), cu(lk)
    G = n1 // n2
    q, k, w = (torch.tensor(c[n], requires_grad=True) for n in ("q", "k", "w"))
    dy = torch.tensor(c["dy"])
    total = q.new_zeros(())
    for b in range(len(lq)):
        for t in range(int(cq[b]), int(cq[b + 1])):
            for h in range(n2):
                rows = torch.tensor(c["idx"][t, h].astype(np.int64)) + int(ck[b])
                ks = k[:, h, :].index_select(0, rows)                              # [topK, D]
                s = torch.relu(q[t, h * G:(h + 1) * G] @ ks.T)                     # [G, topK]
                total = total + (dy[t, h] * (w[t, h * G:(h + 1) * G] @ s)).sum()
    total.backward()
    dq, dk, dw = O.indexer_backward(c["q"], c["k"], c["w"], c["dy"], c["idx"], cq, ck, n1, n2)
    for mine, ref in ((dq, q.grad), (dk, k.grad), (dw, w.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-11, atol=1e-12)


def test_indexer_closed_forms():
    """Weights = 0: Y = 0, so dQ = dK = 0 while dW = sum_k S dy.  All pre-activations negative
    (every selected key is -c times the query): S = 0, so every gradient is 0."""
    rng = np.random.default_rng(34)
    lq, lk, n1, n2, d, topk = (4,), (6,), 2, 1, 3, 3
    c = case(rng, lq, lk, n1, n2, d, topk)
    cq, ck = cu(lq), cu(lk)
    dq, dk, dw = O.indexer_backward(c["q"], c["k"], np.zeros_like(c["w"]), c["dy"], c["idx"], cq, ck, n1, n2)
    assert not dq.any() and not dk.any()
    S = np.maximum(np.einsum("thd,tkd->thk", c["q"], c["k"][c["idx"][:, 0], 0]), 0.0)
    np.testing.assert_allclose(dw, (S * c["dy"][:, 0][:, None, :]).sum(-1), rtol=1e-13)
    q = np.ones((4, n1, d))
    k = -np.ones((6, n2, d)) * 2.0
    dq, dk, dw = O.indexer_backward(q, k, c["w"], c["dy"], c["idx"], cq, ck, n1, n2)
    assert not dq.any() and not dk.any() and not dw.any()
