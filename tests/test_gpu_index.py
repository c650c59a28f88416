"""The inverted index of the selected backward, checked entry by entry (integer work:
bit-exact) against numpy's stable argsort of the topk keys, through the diagnostic export
attn_bwd_selected_index.  Covers the chunked counting-sort path, the atomic-fill-and-sort
fallback, the identity work order above 8192 keys, and out-of-range ids."""
import numpy as np
import pytest
import torch

import sparse_attention_backward_amd as sab
import workloads as W

pytestmark = pytest.mark.gpu


def expected_index(w, topk):
    """offsets, lists and work order of the page's Gather, inverted: key = (KV head, block of
    the token's own sequence), list = ascending entries t * cnt + slot that chose it."""
    T1, n2, cnt = topk.shape
    cu_q, cu_kv = np.asarray(w.cu_q), np.asarray(w.cu_kv)
    nblk = (cu_kv[1:] - cu_kv[:-1]) // w.block_size
    blkoff = np.concatenate([[0], np.cumsum(nblk)])
    NB = int(blkoff[-1])
    seq = np.searchsorted(cu_q, np.arange(T1), side="right") - 1
    e = np.arange(T1 * n2 * cnt, dtype=np.int64)
    t, kvh, slot = e // (n2 * cnt), (e // cnt) % n2, e % cnt
    ids = topk.reshape(-1).astype(np.int64)
    b = seq[t]
    valid = (ids >= 0) & (ids < nblk[b])
    key = kvh * NB + blkoff[b] + ids
    kv, val = key[valid], (t * cnt + slot)[valid]
    lists = val[np.argsort(kv, kind="stable")].astype(np.int32)
    counts = np.bincount(kv, minlength=n2 * NB)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    keys = np.arange(n2 * NB)
    # length classes: thresholds t_0 = longest, t_(k+1) = floor(4 t_k / 5); the least k < 31 with
    # length > t_(k+1), else 31; ordered by class, then key
    longest = int(counts.max(initial=0))

    def length_class(n):
        t = longest
        for k in range(31):
            t = t * 4 // 5
            if n > t:
                return k
        return 31

    cls = np.array([length_class(int(n)) for n in counts], dtype=np.int64)
    order = np.lexsort((keys, cls)).astype(np.int32) if n2 * NB <= 8192 else keys.astype(np.int32)
    return offsets, lists, order, bool((~valid).any())


def run_index(w, topk_dev):
    dev = topk_dev.device
    prob = sab.Problem.selected(w.cu_q, w.cu_kv, w.n1, w.n2, w.d_qk, w.d_v, w.scale, w.block_size, w.block_count)
    ws = torch.empty(max(1, sab.attn_bwd_workspace_size(prob)), dtype=torch.uint8, device=dev)
    nkeys = w.n2 * int(sum((np.asarray(w.seqlens_kv) // w.block_size)))
    offsets = torch.full((nkeys + 1,), -7, dtype=torch.int32, device=dev)
    order = torch.full((nkeys,), -7, dtype=torch.int32, device=dev)
    lists = torch.full((max(1, topk_dev.numel()),), -7, dtype=torch.int32, device=dev)
    sab.attn_bwd_selected_index(prob, topk_dev, offsets, lists, order, ws)
    raised = sab.attn_bwd_check_index_flag(prob, ws)
    return offsets.cpu().numpy(), lists.cpu().numpy(), order.cpu().numpy(), raised


def check(w, topk_dev):
    print(f"[index] {w.name} T1={w.T1} n2={w.n2} cnt={w.block_count} bs={w.block_size}", flush=True)
    off, lst, order, raised = run_index(w, topk_dev)
    e_off, e_lst, e_order, e_raised = expected_index(w, topk_dev.cpu().numpy())
    np.testing.assert_array_equal(off, e_off)
    n = int(e_off[-1])
    np.testing.assert_array_equal(lst[:n], e_lst)
    np.testing.assert_array_equal(order, e_order)
    assert raised == e_raised


def test_index_zipf_varlen_fullsize():
    w = W.config(4)   # Zipf-skewed ids: hot blocks with every token of their sequence
    x = W.make_inputs(w, device="cuda", backend="torch")
    check(w, x["topk"])


def test_index_s32k_fullsize():
    w = W.config(3)
    x = W.make_inputs(w, device="cuda", backend="torch")
    check(w, x["topk"])


@pytest.mark.parametrize("kw", [
    # few entries over many blocks: the atomic-fill-and-sort fallback
    dict(seqlens=(8,), seqlens_kv=(2048,), block_size=16, block_count=2, n1=16, n2=1),
    # more than 16384 keys (LDS histogram limit): fallback path, identity work order
    dict(seqlens=(64,), seqlens_kv=(131072,), block_size=16, block_count=32, n1=16, n2=4),
    # ragged sequences, an empty one, repeated work across KV heads
    dict(seqlens=(200, 0, 64), seqlens_kv=(256, 128, 192), block_size=64, block_count=2, index_dist="zipf"),
])
def test_index_small(kw):
    w = W.small_selected(**kw)
    x = W.make_inputs(w)
    check(w, x["topk"].cuda())


def test_index_out_of_range_ids_are_left_out():
    w = W.small_selected(seqlens=(200, 64), seqlens_kv=(256, 192), block_size=64, block_count=2)
    x = W.make_inputs(w)
    topk = x["topk"].clone()
    topk[3, 0, 1] = 4        # sequence 0 has 4 blocks
    topk[210, 1, 0] = -1     # sequence 1
    topk[250, 0, 1] = 1 << 20
    check(w, topk.cuda())
    off, lst, order, raised = run_index(w, topk.cuda())
    assert raised and off[-1] == topk.numel() - 3
