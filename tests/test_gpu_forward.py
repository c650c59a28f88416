"""GPU parity of the selected forward (attn_fwd_selected), of the selected backward without
attentionOut, and of the fp16 selected path, against the float64 oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_backward_amd as sab
import workloads as W
from helpers import (assert_close, check_against_oracle, f64, gpu_backward, oracle_backward, oracle_forward,
                     problem_for)

pytestmark = pytest.mark.gpu

# fp32 statistics from fp32 accumulation of exact products: the maximum to 1e-3 absolute per
# unit of magnitude, the sum to 1e-3 relative (the scores carry ~1e-5 relative rounding)
STAT_TOL = 1e-3

SHAPES = [
    dict(seqlens=(256, 384), block_size=64, block_count=3),
    dict(seqlens=(256, 512), block_size=128, block_count=2),
    dict(seqlens=(192, 96), block_size=32, block_count=3, n1=16, n2=2),
    dict(seqlens=(128, 128), block_size=16, block_count=5, n1=8, n2=1, d_qk=128, d_v=128),
    dict(seqlens=(96, 64), seqlens_kv=(384, 192), block_size=96, block_count=2, n1=6, n2=2),
    dict(seqlens=(40,), seqlens_kv=(8192,), block_size=128, block_count=63, n1=64, n2=2),   # G = 32
    dict(seqlens=(200, 0, 64), seqlens_kv=(256, 128, 192), block_size=64, block_count=2, index_dist="zipf"),
    dict(seqlens=(1,), seqlens_kv=(64,), block_size=64, block_count=1, n1=16, n2=1),
]


def _gpu_forward(w, x):
    dev = torch.device("cuda", 0)
    g = lambda t: t.to(dev).contiguous()  # noqa: E731
    prob = sab.Problem.selected(w.cu_q, w.cu_kv, w.n1, w.n2, w.d_qk, w.d_v, w.scale, w.block_size, w.block_count,
                                dtype=w.dtype, forward=True)
    ws = torch.empty(max(1, sab.attn_bwd_workspace_size(prob)), dtype=torch.uint8, device=dev)
    out, smax, ssum = sab.selected_forward(prob, g(x["query"]), g(x["key"]), g(x["value"]), g(x["topk"]), ws)
    torch.cuda.synchronize()
    return prob, ws, out, smax, ssum


def _check_stats(name, smax, ssum, m, l):
    smax, ssum = f64(smax), f64(ssum)
    assert (smax == smax[..., :1]).all() and (ssum == ssum[..., :1]).all(), f"{name}: the 8 lanes differ"
    np.testing.assert_array_less(np.abs(smax[..., 0] - m), STAT_TOL * np.maximum(1.0, np.abs(m)) + 1e-30,
                                 err_msg=f"{name}: softmaxMax")
    np.testing.assert_array_less(np.abs(ssum[..., 0] - l), STAT_TOL * np.abs(l) + 1e-30, err_msg=f"{name}: softmaxSum")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("kw", SHAPES)
def test_selected_forward(kw, dtype):
    w = W.small_selected(dtype=dtype, **kw)
    x = W.make_inputs(w)
    print(f"[forward] {w.name} seqlens={w.seqlens_q}/{w.seqlens_kv} n1={w.n1} n2={w.n2} bs={w.block_size} "
          f"cnt={w.block_count}", flush=True)
    prob, ws, out, smax, ssum = _gpu_forward(w, x)
    o, m, l = O.forward_selected(f64(x["query"]), f64(x["key"]), f64(x["value"]), x["topk"].numpy(), w.cu_q,
                                 w.cu_kv, w.n1, w.n2, w.scale, w.block_size)
    assert_close(f"{w.name}:out", f64(out), o, w.dtype)
    _check_stats(w.name, smax, ssum, m, l)
    assert not sab.attn_bwd_check_index_flag(prob, ws)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("kw", SHAPES)
def test_selected_backward_without_out(kw, dtype):
    """attentionOut omitted: rowsum(P dP) from the gathered rows instead of rowsum(dY O)."""
    w = W.small_selected(dtype=dtype, **kw)
    x = W.make_inputs(w)
    print(f"[no-out] {w.name} seqlens={w.seqlens_q}/{w.seqlens_kv} n1={w.n1} n2={w.n2} bs={w.block_size}", flush=True)
    _, smax, ssum = oracle_forward(w, x)
    got = gpu_backward(w, x, None, smax, ssum)
    check_against_oracle(w, got, oracle_backward(w, x))


@pytest.mark.parametrize("kw", SHAPES[:5])
def test_selected_backward_fp16(kw):
    w = W.small_selected(dtype="fp16", **kw)
    x = W.make_inputs(w)
    o, smax, ssum = oracle_forward(w, x)
    got = gpu_backward(w, x, o, smax, ssum)
    check_against_oracle(w, got, oracle_backward(w, x))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_selected_forward_then_backward(dtype):
    """The GPU forward's out and statistics feed the GPU backward: the gradients match the
    oracle's exact gradient (a training step's two halves on the device)."""
    w = W.small_selected(seqlens=(256, 384), block_size=64, block_count=4, index_dist="zipf", dtype=dtype)
    x = W.make_inputs(w)
    _, _, out, smax, ssum = _gpu_forward(w, x)
    got = gpu_backward(w, x, out, smax, ssum)
    check_against_oracle(w, got, oracle_backward(w, x))


def test_selected_forward_out_of_range_id_raises_flag():
    w = W.small_selected(seqlens=(64, 64), block_size=32, block_count=2, n1=16, n2=1)
    x = W.make_inputs(w)
    x["topk"][5, 0, 1] = 99   # sequence 0 has 2 blocks
    prob, ws, out, smax, ssum = _gpu_forward(w, x)
    assert sab.attn_bwd_check_index_flag(prob, ws)
    assert torch.isfinite(out.float()).all()
    # the row's remaining block is its whole key set: compare with the oracle on that block alone
    ids = x["topk"].clone()
    ids[5, 0, 1] = ids[5, 0, 0]
    t5 = np.array([5])
    o1, m1, l1 = O.forward_selected(f64(x["query"]), f64(x["key"]), f64(x["value"]), ids[:, :, :1].numpy(),
                                    w.cu_q, w.cu_kv, w.n1, w.n2, w.scale, w.block_size, tokens=t5)
    assert_close("out-of-range row", f64(out[5]), o1[5], "bf16")
    _check_stats("out-of-range row", smax[5:6], ssum[5:6], m1[5:6], l1[5:6])


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_selected_bsnd_layout_matches_tnd(dtype):
    """BSND inputs are TND inputs with equal lengths: forward and backward give the same bits."""
    B, S1, S2 = 3, 96, 256
    w = W.small_selected(seqlens=(S1,) * B, seqlens_kv=(S2,) * B, block_size=32, block_count=3, n1=16, n2=2,
                         dtype=dtype)
    x = W.make_inputs(w)
    dev = torch.device("cuda", 0)
    g = lambda t: t.to(dev).contiguous()  # noqa: E731
    res = []
    for bsnd in (None, (B, S1, S2)):
        fw = sab.Problem.selected(w.cu_q, w.cu_kv, w.n1, w.n2, w.d_qk, w.d_v, w.scale, w.block_size, w.block_count,
                                  dtype=dtype, forward=True, bsnd=bsnd)
        out, smax, ssum = sab.selected_forward(fw, g(x["query"]), g(x["key"]), g(x["value"]), g(x["topk"]))
        bw = sab.Problem.selected(w.cu_q, w.cu_kv, w.n1, w.n2, w.d_qk, w.d_v, w.scale, w.block_size, w.block_count,
                                  dtype=dtype, bsnd=bsnd)
        grads = sab.selected_backward(bw, g(x["query"]), g(x["key"]), g(x["value"]), out, g(x["dy"]), smax, ssum,
                                      g(x["topk"]))
        torch.cuda.synchronize()
        res.append((out, smax, ssum) + tuple(grads))
    for a, b in zip(*res):
        assert torch.equal(a, b)
    check_against_oracle(w, dict(zip(("dq", "dk", "dv"), res[1][3:])), oracle_backward(w, x))


@pytest.mark.parametrize("window_tokens", [37, 100])
def test_selected_forward_windows_match_single_window(window_tokens):
    """Windows of query tokens (the partials of one window at a time): each entry's partial and
    each token's merge are the same computations, so the bits do not change."""
    w = W.small_selected(seqlens=(256, 130), seqlens_kv=(256, 192), block_size=64, block_count=3, index_dist="zipf")
    x = W.make_inputs(w)
    dev = torch.device("cuda", 0)
    g = lambda t: t.to(dev).contiguous()  # noqa: E731
    res = []
    for wt in (0, window_tokens):
        fw = sab.Problem.selected(w.cu_q, w.cu_kv, w.n1, w.n2, w.d_qk, w.d_v, w.scale, w.block_size, w.block_count,
                                  forward=True, window_tokens=wt)
        res.append(sab.selected_forward(fw, g(x["query"]), g(x["key"]), g(x["value"]), g(x["topk"])))
        torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b)
    o, m, l = O.forward_selected(f64(x["query"]), f64(x["key"]), f64(x["value"]), x["topk"].numpy(), w.cu_q,
                                 w.cu_kv, w.n1, w.n2, w.scale, w.block_size)
    assert_close(f"{w.name}:out windows", f64(res[1][0]), o, w.dtype)
    _check_stats(w.name, res[1][1], res[1][2], m, l)


def test_selected_backward_without_out_windows_match_single_window():
    """The row statistic without attentionOut runs over the backward's windows: its sums do not
    depend on them, so dQ keeps its bits; dK / dV differ only by the fp32 order of the windows'
    partial sums."""
    w = W.small_selected(seqlens=(256, 130), seqlens_kv=(256, 192), block_size=64, block_count=3)
    x = W.make_inputs(w)
    _, smax, ssum = oracle_forward(w, x)
    a = gpu_backward(w, x, None, smax, ssum, deterministic=True)
    b = gpu_backward(w, x, None, smax, ssum, deterministic=True, window_tokens=41)
    assert torch.equal(a["dq"], b["dq"])
    for n in ("dk", "dv"):
        d = (a[n].double() - b[n].double()).abs().max().item()
        assert d <= 1e-2 * a[n].double().abs().max().item(), (n, d)
    check_against_oracle(w, b, oracle_backward(w, x))
