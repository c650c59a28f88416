"""GPU parity: the HIP library against the float64 oracle, element by element,
on seeded inputs that span several tiles and a ragged tail."""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import (assert_close, check_against_oracle, f64, gpu_backward, oracle_backward, oracle_forward)

pytestmark = pytest.mark.gpu


def _run(w, deterministic=None, dq_mode=0, window_tokens=0):
    x = W.make_inputs(w)
    o, smax, ssum = oracle_forward(w, x)
    print(f"[parity] {w.name} seqlens={w.seqlens_q}/{w.seqlens_kv} n1={w.n1} n2={w.n2} dq_mode={dq_mode} "
          f"window_tokens={window_tokens}", flush=True)
    got = gpu_backward(w, x, o, smax, ssum, deterministic=deterministic, dq_mode=dq_mode, window_tokens=window_tokens)
    ref = oracle_backward(w, x)
    check_against_oracle(w, got, ref)
    return x, got, ref


def test_dense_fp32_config1():
    _run(W.config(1))


# dq_mode 1: dQ from the dS tiles stored by the KV-major pass; 2: dQ recomputed query-major
@pytest.mark.parametrize("dq_mode", [1, 2])
@pytest.mark.parametrize("seqlens,n1,n2,d_qk,d_rope,d_v", [
    ((200, 130), 8, 2, 128, 64, 128),     # rope split, GQA G=4, ragged tails
    ((64, 1, 129), 4, 4, 128, 0, 128),    # no rope, G=1, a one-token sequence
    ((97,), 4, 1, 64, 0, 64),             # small head dim, G=4
    ((300, 64), 16, 2, 128, 64, 128),     # G=8: two passes of four heads in the dQ product
    ((190,), 6, 3, 128, 64, 128),         # G=2
])
def test_dense_bf16_causal(seqlens, n1, n2, d_qk, d_rope, d_v, dq_mode):
    _run(W.small_dense(seqlens=seqlens, n1=n1, n2=n2, d_qk=d_qk, d_rope=d_rope, d_v=d_v), dq_mode=dq_mode)


@pytest.mark.parametrize("dq_mode", [1, 2])
def test_dense_bf16_noncausal_unequal_lengths(dq_mode):
    w = W.small_dense(seqlens=(150,), n1=4, n2=2, d_qk=128, d_rope=64, d_v=128, causal=False)
    w = w.with_(seqlens_q=(150, 0, 70, 33), seqlens_kv=(77, 64, 200, 0), name="dense-noncausal-unequal")
    _run(w, dq_mode=dq_mode)


# Masks on the relative position (causal aligned top-left or bottom-right when the lengths
# differ, windows of pre / next tokens): blocks skipped, blocks crossing an edge masked per
# element, rows that see no key (zero gradients), keys no row sees (zero dK / dV).
MASKS = [
    dict(seqlens=(150, 70), seqlens_kv=(200, 70), causal=True, mask_align=1),       # S1 < S2, bottom-right
    dict(seqlens=(200, 64), seqlens_kv=(90, 64), causal=True, mask_align=1),        # S1 > S2: keyless rows
    dict(seqlens=(120,), seqlens_kv=(210,), causal=True, mask_align=0),             # top-left, S1 < S2
    dict(seqlens=(190, 77), causal=False, band=(40, 5)),                            # window, equal lengths
    dict(seqlens=(130, 96), seqlens_kv=(160, 50), causal=False, band=(17, 33), mask_align=1),
    dict(seqlens=(140,), seqlens_kv=(100,), causal=False, band=(0, 0)),              # the diagonal only
    dict(seqlens=(100,), causal=False, band=(5, -3), mask_align=1),                  # a window off the diagonal
]


@pytest.mark.parametrize("dq_mode", [1, 2])
@pytest.mark.parametrize("kw", MASKS)
def test_dense_bf16_masks(kw, dq_mode):
    _run(W.small_dense(n1=8, n2=2, **kw), dq_mode=dq_mode)


@pytest.mark.parametrize("kw", MASKS[:2] + MASKS[4:5])
def test_dense_fp32_masks(kw):
    _run(W.small_dense(n1=4, n2=2, d_qk=64, d_rope=32, d_v=64, dtype="fp32", **kw))


def test_dense_fp32_small_rope():
    w = W.small_dense(seqlens=(70, 33), n1=4, n2=2, d_qk=64, d_rope=32, d_v=64, dtype="fp32")
    _run(w)


@pytest.mark.parametrize("kw", [
    dict(seqlens=(256, 384), block_size=64, block_count=3),
    dict(seqlens=(256, 512), block_size=128, block_count=2),
    dict(seqlens=(192, 96), block_size=32, block_count=3, n1=16, n2=2),
    dict(seqlens=(128, 128), block_size=16, block_count=5, n1=8, n2=1, d_qk=128, d_v=128),
    dict(seqlens=(200, 0, 64), seqlens_kv=(256, 128, 192), block_size=64, block_count=2, index_dist="zipf"),
    # largest group and gathered length the problem allows: G = 32, cnt * bs = 8064 < 8192
    dict(seqlens=(40,), seqlens_kv=(8192,), block_size=128, block_count=63, n1=64, n2=2),
    # G = 3 (steps of 21 tokens and a padding row); blocks of 96 keys (a partly used 128-key tile)
    dict(seqlens=(96, 64), seqlens_kv=(384, 192), block_size=96, block_count=2, n1=6, n2=2),
    # G = 12 with 32-key blocks
    dict(seqlens=(70,), seqlens_kv=(256,), block_size=32, block_count=4, n1=24, n2=2),
    # few entries over many blocks: the index build takes its atomic-fill-and-sort path
    dict(seqlens=(8,), seqlens_kv=(2048,), block_size=16, block_count=2, n1=16, n2=1),
    # one query token against G = 16 heads and a 64-key block; single-block sequence
    dict(seqlens=(1,), seqlens_kv=(64,), block_size=64, block_count=1, n1=16, n2=1),
])
def test_selected(kw):
    _run(W.small_selected(**kw))


# Windows of query tokens: the dQ shares are formed and summed one window at a time and the
# dK / dV accumulators carried between windows in fp32.  Ragged windows (the last shorter), a
# window shorter than a step's entries, windows that cross a sequence boundary, and blocks
# that no token of a middle window selected.
@pytest.mark.parametrize("window_tokens,kw", [
    (37, dict(seqlens=(256, 384), block_size=64, block_count=3)),
    (100, dict(seqlens=(256, 512), block_size=128, block_count=2)),
    (3, dict(seqlens=(40, 9), seqlens_kv=(512, 256), block_size=64, block_count=2, n1=16, n2=1)),
    (64, dict(seqlens=(200, 0, 64), seqlens_kv=(256, 128, 192), block_size=64, block_count=2, index_dist="zipf")),
    (50, dict(seqlens=(96, 64), seqlens_kv=(384, 192), block_size=96, block_count=2, n1=6, n2=2)),
])
def test_selected_windows(window_tokens, kw):
    _run(W.small_selected(**kw), window_tokens=window_tokens)


def test_selected_windows_match_single_window():
    """dQ does not depend on the windows (same shares, same slot order); dK / dV only through
    the fp32 summation order."""
    w = W.small_selected(seqlens=(256, 384), block_size=64, block_count=4, index_dist="zipf")
    x = W.make_inputs(w)
    o, smax, ssum = oracle_forward(w, x)
    a = gpu_backward(w, x, o, smax, ssum, deterministic=True)
    b = gpu_backward(w, x, o, smax, ssum, deterministic=True, window_tokens=41)
    assert torch.equal(a["dq"], b["dq"])
    for n in ("dk", "dv"):
        d = (a[n].double() - b[n].double()).abs().max().item()
        assert d <= 1e-2 * a[n].double().abs().max().item(), (n, d)


def test_selected_duplicate_ids():
    w = W.small_selected(seqlens=(128, 192), block_size=64, block_count=2)
    x = W.make_inputs(w)
    x["topk"][::3, :, 1] = x["topk"][::3, :, 0]   # literal Gather: a repeated block counts twice
    o, smax, ssum = oracle_forward(w, x)
    got = gpu_backward(w, x, o, smax, ssum)
    check_against_oracle(w, got, oracle_backward(w, x))


def test_selected_deterministic_bitwise():
    w = W.small_selected(seqlens=(256, 384), block_size=64, block_count=4, index_dist="zipf")
    x = W.make_inputs(w)
    o, smax, ssum = oracle_forward(w, x)
    a = gpu_backward(w, x, o, smax, ssum, deterministic=True)
    b = gpu_backward(w, x, o, smax, ssum, deterministic=True)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_dense_deterministic_bitwise():
    w = W.small_dense(seqlens=(300, 77))
    x = W.make_inputs(w)
    o, smax, ssum = oracle_forward(w, x)
    a = gpu_backward(w, x, o, smax, ssum, deterministic=True)
    b = gpu_backward(w, x, o, smax, ssum, deterministic=True)
    for n in a:
        if a[n] is not None:
            assert torch.equal(a[n], b[n]), n


def test_selected_gradient_sums_on_gpu_outputs():
    """rowsum(dS) = 0 => sum_j dK_j = 0 per (sequence, KV head); sum_j dV_j = sum of dY over the group."""
    w = W.small_selected(seqlens=(256, 384), block_size=64, block_count=3)
    x, got, ref = _run(w)
    dk, dv, dy = f64(got["dk"]), f64(got["dv"]), f64(x["dy"])
    G = w.G
    for b in range(w.batch):
        ks, ke = w.cu_kv[b], w.cu_kv[b + 1]
        qs, qe = w.cu_q[b], w.cu_q[b + 1]
        for h in range(w.n2):
            sk = dk[ks:ke, h].sum(axis=0)
            assert np.abs(sk).max() <= 2e-2 * np.abs(dk[ks:ke, h]).sum(axis=0).max() + 1e-6
            want = dy[qs:qe, h * G:(h + 1) * G].sum(axis=(0, 1))
            np.testing.assert_allclose(dv[ks:ke, h].sum(axis=0), want, rtol=2e-2, atol=2e-2 * np.abs(want).max())


def test_selected_out_of_range_id_raises_flag_and_spares_other_rows():
    """An out-of-range id is skipped by every kernel (no contribution) and raises the flag that
    attn_bwd_check_index_flag reads.  dQ rows of the other tokens are unaffected and match the
    oracle (which is given a valid id in that slot: dQ of a token depends on its own ids only)."""
    import sparse_attention_backward_amd as sab
    w = W.small_selected(seqlens=(128, 64), seqlens_kv=(256, 192), block_size=64, block_count=2, n1=16, n2=2)
    x = W.make_inputs(w)
    bad = x["topk"].clone()
    bad[7, 1, 0] = 4          # sequence 0 has 4 blocks
    dev = torch.device("cuda", 0)
    o, smax, ssum = oracle_forward(w, x)
    prob = sab.Problem.selected(w.cu_q, w.cu_kv, w.n1, w.n2, w.d_qk, w.d_v, w.scale, w.block_size, w.block_count)
    ws = torch.empty(sab.attn_bwd_workspace_size(prob), dtype=torch.uint8, device=dev)
    g = lambda t: t.to(dev).contiguous()  # noqa: E731
    dq, dk, dv = sab.selected_backward(prob, g(x["query"]), g(x["key"]), g(x["value"]), g(o), g(x["dy"]), g(smax),
                                       g(ssum), g(bad), workspace=ws)
    torch.cuda.synchronize()
    assert sab.attn_bwd_check_index_flag(prob, ws)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    ref = oracle_backward(w, x)
    keep = np.ones(w.T1, dtype=bool)
    keep[7] = False
    assert_close("other tokens' dq", f64(dq)[keep], ref["dq"][keep], "bf16")
    # a clean call on the same workspace clears the flag
    sab.selected_backward(prob, g(x["query"]), g(x["key"]), g(x["value"]), g(o), g(x["dy"]), g(smax), g(ssum),
                          g(x["topk"]), workspace=ws)
    torch.cuda.synchronize()
    assert not sab.attn_bwd_check_index_flag(prob, ws)
