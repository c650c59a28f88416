"""GPU parity of the lightning-indexer backward (attn_bwd_indexer) against the float64 oracle
(oracle/indexer.py), in its three modes: ordered dK sums (deterministic 0 or 1) and fp32
atomics (dk_atomic).

The ReLU mask is a decision taken on S: the kernel forms S in fp32 from bf16 inputs, the
oracle in float64, so a score within rounding of 0 could fall on different sides.  Such
(token, key head, slot) entries -- any head with |S| below 1e-3 in float64 -- get dy = 0 in
these tests, so that neither side's result depends on the side its S fell (R and S dy are
0 for them in both)."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_backward_amd as sab
import workloads as W
from helpers import assert_close, assert_rows_close, f64

pytestmark = pytest.mark.gpu

EDGE = 1e-3


def _inputs(w):
    x = W.make_indexer_inputs(w)
    q, k, idx = f64(x["q"]), f64(x["k"]), x["indices"].numpy()
    cu_q, cu_kv = w.cu_q, w.cu_kv
    dy = x["dy"].clone()
    seq = np.searchsorted(cu_q, np.arange(w.T1), side="right") - 1
    for t in range(w.T1):
        for h in range(w.n2):
            rows = cu_kv[seq[t]] + idx[t, h].astype(np.int64)
            valid = (idx[t, h] >= 0) & (idx[t, h] < cu_kv[seq[t] + 1] - cu_kv[seq[t]])
            S = q[t, h * w.G:(h + 1) * w.G] @ k[np.where(valid, rows, 0), h].T
            near = (np.abs(S) < EDGE).any(axis=0) & valid
            dy[t, h, torch.from_numpy(near)] = 0
    x["dy"] = dy
    return x


def _run(w, deterministic, window_tokens=0, x=None, dk_atomic=False):
    x = x if x is not None else _inputs(w)
    dev = torch.device("cuda", 0)
    g = lambda t: t.to(dev).contiguous()  # noqa: E731
    prob = sab.Problem.indexer(w.cu_q, w.cu_kv, w.n1, w.n2, w.topk, deterministic=deterministic,
                               window_tokens=window_tokens, dk_atomic=dk_atomic)
    ws = torch.empty(max(1, sab.attn_bwd_workspace_size(prob)), dtype=torch.uint8, device=dev)
    print(f"[indexer] seqlens={w.seqlens_q}/{w.seqlens_kv} n1={w.n1} n2={w.n2} topk={w.topk} "
          f"det={deterministic} atomic={dk_atomic} window_tokens={window_tokens}", flush=True)
    dq, dk, dw = sab.indexer_backward(prob, g(x["q"]), g(x["k"]), g(x["weights"]), g(x["dy"]), g(x["indices"]), ws)
    torch.cuda.synchronize()
    return x, (dq, dk, dw), sab.attn_bwd_check_index_flag(prob, ws)


def _check(w, x, got):
    rq, rk, rw = O.indexer_backward(f64(x["q"]), f64(x["k"]), f64(x["weights"]), f64(x["dy"]), x["indices"].numpy(),
                                    w.cu_q, w.cu_kv, w.n1, w.n2)
    dq, dk, dw = got
    assert_close("indexer dq", f64(dq), rq, "bf16")
    assert_rows_close("indexer dq rows", f64(dq), rq, "bf16")
    assert_close("indexer dk", f64(dk), rk, "bf16")
    assert_close("indexer dw", f64(dw), rw, "bf16")


SHAPES = [
    dict(seqlens=(96, 64), seqlens_kv=(160, 130), n1=16, n2=1, topk=40),     # ragged last chunk of keys
    dict(seqlens=(70,), seqlens_kv=(300,), n1=64, n2=2, topk=64),            # G = 32
    dict(seqlens=(33, 0, 40), seqlens_kv=(200, 64, 128), n1=64, n2=1, topk=128),   # G = 64, an empty sequence
    dict(seqlens=(50,), seqlens_kv=(96,), n1=10, n2=2, topk=96),             # G = 5 (padding heads), every key
]


@pytest.mark.parametrize("mode", ["default", "deterministic", "atomic"])
@pytest.mark.parametrize("kw", SHAPES)
def test_indexer(kw, mode):
    w = W.small_indexer(**kw)
    x, got, raised = _run(w, mode == "deterministic", dk_atomic=mode == "atomic")
    assert not raised
    _check(w, x, got)


def test_indexer_deterministic_windows_and_bitwise_repeat():
    w = W.small_indexer(seqlens=(96, 64), seqlens_kv=(160, 130), n1=32, n2=2, topk=48)
    x = _inputs(w)
    _, a, _ = _run(w, True, window_tokens=37, x=x)
    _, b, _ = _run(w, True, window_tokens=37, x=x)
    _, c, _ = _run(w, True, x=x)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    assert torch.equal(a[0], c[0]) and torch.equal(a[2], c[2])   # dQ, dW do not depend on the windows
    _check(w, x, a)


def test_indexer_repeated_and_out_of_range_indices():
    w = W.small_indexer(seqlens=(40,), seqlens_kv=(100,), n1=16, n2=1, topk=32)
    x = _inputs(w)
    x["indices"][::3, 0, 5] = x["indices"][::3, 0, 4]     # a repeated index counts twice
    _, got, raised = _run(w, True, x=x)
    assert not raised
    _check(w, x, got)
    bad = {k: v.clone() for k, v in x.items()}
    bad["indices"][7, 0, 3] = 100                          # sequence of 100 keys
    for det, atomic in ((False, True), (True, False)):
        _, got, raised = _run(w, det, x=bad, dk_atomic=atomic)
        assert raised
        for t in got:
            assert torch.isfinite(t.float()).all()
