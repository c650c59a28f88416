"""C-ABI boundary on the CPU: the library loads, exports every function the header
declares, and maps each constraint of the pages to its status code before touching
any device (no kernel is launched by these tests)."""
import ctypes
import math
import os
import re

import pytest

import sparse_attention_backward_amd as sab
import workloads as W

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "attn_bwd.h")

OK, NULLPTR, INVALID, UNSUPPORTED, WORKSPACE = (sab.ATTN_OK, sab.ATTN_ERR_NULLPTR, sab.ATTN_ERR_INVALID,
                                                sab.ATTN_ERR_UNSUPPORTED, sab.ATTN_ERR_WORKSPACE)
FAKE = 0x10000  # a 256-byte aligned non-null address; never dereferenced by the failing paths below


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:attn_status_t|const char\*)\s+(attn_(?:bwd|fwd)_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    fns = header_functions()
    for name in ("attn_bwd_workspace_size", "attn_bwd_dense_varlen", "attn_bwd_selected"):
        assert name in fns


def test_library_exports_every_declared_function():
    L = ctypes.CDLL(sab.LIB_PATH)
    for name in header_functions():
        assert hasattr(L, name), name
    assert set(header_functions()) == set(sab.EXPORTED_SYMBOLS)


def status_ws(prob):
    n = ctypes.c_uint64(0)
    return sab.lib.attn_bwd_workspace_size(prob.ref, ctypes.byref(n)), n.value


def dense(**kw):
    base = dict(cu_q=[0, 100, 164], cu_kv=[0, 100, 164], n1=8, n2=2, d_qk=128, d_v=128, scale=0.1, causal=True,
                d_rope=64, dtype="bf16")
    base.update(kw)
    return sab.Problem.dense(base.pop("cu_q"), base.pop("cu_kv"), base.pop("n1"), base.pop("n2"), base.pop("d_qk"),
                             base.pop("d_v"), base.pop("scale"), **base)


def selected(**kw):
    base = dict(cu_q=[0, 256, 640], cu_kv=[0, 256, 640], n1=32, n2=2, d_qk=192, d_v=128, scale=0.07,
                block_size=64, block_count=3)
    base.update(kw)
    return sab.Problem.selected(base.pop("cu_q"), base.pop("cu_kv"), base.pop("n1"), base.pop("n2"),
                                base.pop("d_qk"), base.pop("d_v"), base.pop("scale"), base.pop("block_size"),
                                base.pop("block_count"), **base)


@pytest.mark.parametrize("i", W.CONFIGS)
def test_the_five_workloads_validate(i):
    w = W.config(i)
    from helpers import problem_for
    st, n = status_ws(problem_for(w))
    assert st == OK and n > 0


def test_version_and_status_strings():
    assert re.match(r"^\d+\.\d+\.\d+$", sab.attn_bwd_version())
    for s in range(6):
        assert sab.attn_bwd_status_string(s)


def test_null_arguments():
    n = ctypes.c_uint64(0)
    assert sab.lib.attn_bwd_workspace_size(None, ctypes.byref(n)) == NULLPTR
    assert sab.lib.attn_bwd_workspace_size(dense().ref, None) == NULLPTR
    p = dense()
    p.s.cu_seqlens_q = ctypes.cast(None, ctypes.POINTER(ctypes.c_int64))
    assert status_ws(p)[0] == NULLPTR


@pytest.mark.parametrize("kw,want", [
    (dict(), OK),
    (dict(d_qk=100), INVALID),                              # D multiple of 8
    (dict(d_v=12), INVALID),
    (dict(d_v=192, d_qk=128), INVALID),                     # value D <= query D
    (dict(n1=6, n2=4), INVALID),                            # Nq / Nkv integer
    (dict(n1=512, n2=2), INVALID),                          # N <= 256
    (dict(d_qk=512, d_rope=512), INVALID),                  # D <= 768
    (dict(cu_q=[0, 100, 160], cu_kv=[0, 100, 164]), OK),   # causal with unequal lengths: aligned
    (dict(cu_q=[0, 100, 160], cu_kv=[0, 100, 164], align=1), OK),
    (dict(align=2), INVALID),
    (dict(causal=False, band=(16, 0)), OK),                 # window of pre / next tokens
    (dict(causal=False, band=(-3, 2), align=1), INVALID),   # empty window: pre + next < 0
    (dict(causal=False, band=(3, -2)), OK),
    (dict(causal=True, band=(16, 0)), INVALID),             # causal and window exclude each other
    (dict(causal=False, band=((1 << 30) + 1, 0)), INVALID),
    (dict(cu_q=[1, 100, 164]), INVALID),                    # cu starts at 0
    (dict(cu_q=[0, 100, 90], cu_kv=[0, 100, 90]), INVALID),  # non-decreasing
    (dict(cu_q=[0, (1 << 20) + 1], cu_kv=[0, (1 << 20) + 1]), INVALID),  # T <= 1M
    (dict(dtype="fp16"), UNSUPPORTED),
    (dict(d_qk=96, d_rope=0, d_v=96), UNSUPPORTED),         # valid, no bf16 kernel built for 96/96
    (dict(dtype="fp32", d_qk=64, d_rope=32, d_v=64), OK),
    (dict(dtype="fp32", d_qk=256, d_rope=64, d_v=64), UNSUPPORTED),
    (dict(scale=math.nan), INVALID),
    (dict(causal=False, cu_q=[0, 5, 5], cu_kv=[0, 0, 9]), OK),  # zero-length sequences are allowed
])
def test_dense_constraints(kw, want):
    assert status_ws(dense(**kw))[0] == want


@pytest.mark.parametrize("kw,want", [
    (dict(), OK),
    (dict(block_size=40), INVALID),                         # multiple of 16
    (dict(block_size=256, cu_q=[0, 512], cu_kv=[0, 512]), INVALID),  # <= 128
    (dict(block_count=0), INVALID),
    (dict(block_count=129, block_size=16, cu_q=[0, 4096], cu_kv=[0, 4096]), INVALID),
    (dict(block_count=64, block_size=128, cu_q=[0, 8192], cu_kv=[0, 8192]), INVALID),  # count*size < 8K
    (dict(cu_q=[0, 256, 640], cu_kv=[0, 256, 650]), INVALID),  # S2 multiple of block size
    (dict(cu_q=[0, 256, 640], cu_kv=[0, 128, 512]), INVALID),  # S2 >= count*size
    (dict(cu_q=[0, 0, 640], cu_kv=[0, 64, 448]), OK),        # a sequence without queries may be short
    (dict(d_qk=64), INVALID),                                # D in {128, 192}
    (dict(d_v=64), INVALID),
    (dict(n1=64, n2=1), INVALID),                            # G <= 32
    (dict(n1=256, n2=8), INVALID),                           # N1 <= 128
    (dict(n1=7, n2=2), INVALID),
    (dict(n1=64, n2=2), OK),                                 # G = 32, the largest group
    (dict(d_v=192), UNSUPPORTED),                            # 192/192: valid, not built
    (dict(dtype="fp16"), OK),                                 # FLOAT16 (parameter table)
    (dict(dtype="fp32"), INVALID),                           # not a dtype of the selected page
    (dict(cu_q=[0, 256, 640 + (128 << 10)], cu_kv=[0, 256, 640 + (128 << 10)]), INVALID),  # S <= 128K
])
def test_selected_constraints(kw, want):
    assert status_ws(selected(**kw))[0] == want


def test_selected_rejects_rope_and_causal():
    p = selected()
    p.s.d_rope = 64
    assert status_ws(p)[0] == INVALID
    p = selected()
    p.s.causal = 1
    assert status_ws(p)[0] == INVALID


def test_selected_pointers():
    p = selected()
    n = sab.attn_bwd_workspace_size(p)
    L = sab.lib
    args = [FAKE] * 11
    # out == NULL is allowed (attentionOut is optional); the other inputs are required
    a = list(args); a[7] = None   # topk
    assert L.attn_bwd_selected(p.ref, *a, FAKE, n, None) == NULLPTR
    assert L.attn_bwd_selected(p.ref, *args, None, n, None) == WORKSPACE
    assert L.attn_bwd_selected(p.ref, *args, FAKE, n - 1, None) == WORKSPACE
    a = list(args); a[0] = FAKE + 2  # misaligned query
    assert L.attn_bwd_selected(p.ref, *a, FAKE, n, None) == INVALID


def test_dense_pointer_rules():
    p = dense()
    n = sab.attn_bwd_workspace_size(p)
    L = sab.lib
    full = [FAKE] * 14
    a = list(full); a[1] = None   # q_rope missing while d_rope > 0
    assert L.attn_bwd_dense_varlen(p.ref, *a, FAKE, n, None) == NULLPTR
    p0 = dense(d_rope=0)
    n0 = sab.attn_bwd_workspace_size(p0)
    # rope pointers must be NULL when d_rope == 0
    assert L.attn_bwd_dense_varlen(p0.ref, *full, FAKE, n0, None) == INVALID
    assert L.attn_bwd_dense_varlen(p.ref, *full, FAKE + 64, n, None) == WORKSPACE   # workspace alignment 256


def test_empty_batch_is_a_noop():
    p = dense(cu_q=[0, 0], cu_kv=[0, 0], causal=True)
    st, n = status_ws(p)
    assert st == OK
    L = sab.lib
    assert L.attn_bwd_dense_varlen(p.ref, *([None] * 14), FAKE, n, None) == OK


def test_workspace_grows_with_the_problem():
    a = status_ws(selected())[1]
    b = status_ws(selected(cu_q=[0, 512, 1280], cu_kv=[0, 512, 1280]))[1]
    assert b > a


def test_dense_dq_mode_field():
    assert status_ws(dense(dq_mode=3))[0] == INVALID
    assert status_ws(dense(dq_mode=-1))[0] == INVALID
    st1, n1 = status_ws(dense(dq_mode=1))
    st2, n2 = status_ws(dense(dq_mode=2))
    st0, n0 = status_ws(dense())
    assert st0 == st1 == st2 == OK
    # stored dS: causal (query tile, key tile) blocks of the two sequences (lengths 100 and 64:
    # 2 and 1 tiles of 64 -> 3 + 1 blocks), 8 heads, 8 KiB each
    assert n1 - n2 == (3 + 1) * 8 * 64 * 64 * 2
    assert n0 == n1  # small problems store dS
    p = selected()
    p.s.dense_dq_mode = 1
    assert status_ws(p)[0] == INVALID


# ---- selected workspace bound -------------------------------------------------------------
SHARE_CAP = 64 << 30   # dQ shares of one window: at most 64 GiB (then more windows)


def _selected_ws_bound(T1, T2, n1, n2, d_qk, d_v, bs, cnt):
    """Workspace the selected call may take: the share cap plus terms linear in the inputs --
    12 B per topk entry (list, sort scratch), the per-block fp32 dK / dV sums carried between
    windows (at most 64 / 128 keys per block), the row statistics (8 B per query row) and the
    index tables (12 B per block and KV head), with 1 MiB of slack for tables and alignment."""
    entries = T1 * n2 * cnt
    keys = n2 * (T2 // bs)
    kb = 128 if bs > 64 else 64
    return SHARE_CAP + 12 * entries + 4 * keys * kb * (d_qk + d_v) + 8 * T1 * n1 + 12 * keys + (1 << 20)


@pytest.mark.parametrize("S,n1,n2,bs,cnt,d_qk,d_v", [
    (128 << 10, 128, 4, 16, 128, 192, 128),      # longest sequence, most heads, most blocks of the smallest size
    (128 << 10, 128, 128, 64, 64, 192, 128),      # G = 1
    (128 << 10, 64, 2, 128, 63, 192, 128),        # cnt * bs = 8064, the largest gather
    (128 << 10, 96, 3, 32, 100, 128, 128),
])
def test_selected_workspace_bounded_at_extreme_shapes(S, n1, n2, bs, cnt, d_qk, d_v):
    entries = S * n2 * cnt
    p = selected(cu_q=[0, S], cu_kv=[0, S], n1=n1, n2=n2, d_qk=d_qk, d_v=d_v, block_size=bs, block_count=cnt)
    st, n = status_ws(p)
    if entries >= 1 << 31:   # list entries are 32-bit: such problems are refused, not mis-sized
        assert st == UNSUPPORTED
        return
    assert st == OK
    assert n <= _selected_ws_bound(S, S, n1, n2, d_qk, d_v, bs, cnt), n
    full_shares = S * cnt * n1 * d_qk * 2
    if full_shares > SHARE_CAP:
        assert n < full_shares  # the shares of the whole problem would not fit: windows


def test_selected_window_tokens_shrink_the_workspace():
    big = status_ws(selected())[1]
    small = status_ws(selected(window_tokens=16))[1]
    assert small < big
    assert status_ws(selected(window_tokens=-1))[0] == INVALID
    d = dense()
    d.s.sel_window_tokens = 5   # a selected-only field: must be 0 for dense problems
    assert status_ws(d)[0] == INVALID


def test_noalloc_refuses_problems_beyond_the_scratch_array_on_the_host():
    """The size check of attn_bwd_dense_varlen_noalloc runs before any device call."""
    p = dense(cu_q=[0, 300000], cu_kv=[0, 300000], n1=32, n2=8, dq_mode=2)
    st, n = status_ws(p)
    assert st == OK and n > sab.NOALLOC_SCRATCH_BYTES
    args = [FAKE] * 14
    assert sab.lib.attn_bwd_dense_varlen_noalloc(p.ref, *args, None) == WORKSPACE


def test_selected_forward_validation():
    """attn_fwd_selected: op ATTN_OP_SELECTED_FWD, the selected constraints, a workspace of the
    inverted index and one partial per (entry, head): d_v elements + (m_b, l_b)."""
    fw = selected(forward=True)
    st, n = status_ws(fw)
    T1, cnt, n1, n2, d_v = 640, 3, 32, 2, 128
    partials = T1 * cnt * n1 * (2 * d_v + 8)
    index = 12 * T1 * n2 * cnt            # list and sort scratch
    assert st == OK and partials + index <= n <= partials + index + (1 << 16)
    small = selected(forward=True, window_tokens=100)
    assert status_ws(small)[1] < n        # windows of query tokens bound the partials
    assert status_ws(selected(forward=True, block_size=24))[0] == INVALID
    L = sab.lib
    args = [FAKE] * 7
    assert L.attn_fwd_selected(selected().ref, *args, FAKE, n, None) == INVALID      # backward problem
    a = list(args); a[3] = None   # topk
    assert L.attn_fwd_selected(fw.ref, *a, FAKE, n, None) == NULLPTR
    assert L.attn_fwd_selected(fw.ref, *args, FAKE, n - 1, None) == WORKSPACE
    a = list(args); a[4] = FAKE + 4  # misaligned out
    assert L.attn_fwd_selected(fw.ref, *a, FAKE, n, None) == INVALID


def test_bsnd_layout_is_tnd_with_equal_lengths():
    """BSND ([B, S, N, D], the non-TND layout of the selected page): the same workspace as
    the TND problem with B sequences of S queries and S2 keys; TND only for the dense form."""
    B, S1, S2 = 3, 192, 256
    cu_q, cu_kv = [b * S1 for b in range(B + 1)], [b * S2 for b in range(B + 1)]
    tnd = selected(cu_q=cu_q, cu_kv=cu_kv)
    bsnd = selected(cu_q=[0], cu_kv=[0], bsnd=(B, S1, S2))
    assert status_ws(bsnd) == status_ws(tnd)
    fw = selected(cu_q=[0], cu_kv=[0], bsnd=(B, S1, S2), forward=True)
    assert status_ws(fw)[0] == OK
    d = dense()
    d.s.layout = sab.ATTN_LAYOUT_BSND
    d.s.cu_seqlens_q = ctypes.cast(None, ctypes.POINTER(ctypes.c_int64))
    d.s.cu_seqlens_kv = ctypes.cast(None, ctypes.POINTER(ctypes.c_int64))
    d.s.seq_len_q = d.s.seq_len_kv = 64
    assert status_ws(d)[0] == INVALID
    bad = selected(cu_q=[0], cu_kv=[0], bsnd=(B, S1, S2))
    bad.s.cu_seqlens_q = tnd.s.cu_seqlens_q        # BSND takes no sequence offsets
    assert status_ws(bad)[0] == INVALID
    t2 = selected(cu_q=cu_q, cu_kv=cu_kv)
    t2.s.seq_len_q = 5                             # TND takes no BSND lengths
    assert status_ws(t2)[0] == INVALID
    t3 = selected(cu_q=cu_q, cu_kv=cu_kv)
    t3.s.layout = 7
    assert status_ws(t3)[0] == INVALID


def test_mask_fields_are_dense_only():
    for field, val in (("band", 1), ("mask_align", 1), ("pre_tokens", 3), ("next_tokens", 3)):
        p = selected()
        setattr(p.s, field, val)
        assert status_ws(p)[0] == INVALID, field
    d = dense(causal=False)
    d.s.pre_tokens = 4   # window sizes without the window flag
    assert status_ws(d)[0] == INVALID


def _indexer(**kw):
    base = dict(cu_q=[0, 96, 160], cu_kv=[0, 160, 290], n1=16, n2=1, topk=40)
    base.update(kw)
    return sab.Problem.indexer(base.pop("cu_q"), base.pop("cu_kv"), base.pop("n1"), base.pop("n2"), base.pop("topk"),
                               **base)


def test_indexer_validation():
    assert status_ws(_indexer())[0] == OK
    assert status_ws(_indexer(topk=200))[0] == INVALID            # a sequence holds fewer keys than topK
    assert status_ws(_indexer(d=64))[0] == UNSUPPORTED           # D = 128 only
    assert status_ws(_indexer(n1=128, n2=1))[0] == INVALID       # G <= 64
    assert status_ws(_indexer(n1=6, n2=4))[0] == INVALID
    p = _indexer()
    p.s.block_size = 2
    assert status_ws(p)[0] == INVALID                            # one key per index
    p = _indexer()
    p.s.dtype = sab.ATTN_FP16
    assert status_ws(p)[0] == UNSUPPORTED
    small = status_ws(_indexer(window_tokens=8))[1]
    big = status_ws(_indexer())[1]
    atomic = status_ws(_indexer(dk_atomic=True))[1]
    assert atomic < small < big                                  # the shares buffer is per window
    assert status_ws(_indexer(deterministic=True))[1] == big
    assert status_ws(_indexer(deterministic=True, dk_atomic=True))[1] == big   # atomics off when deterministic
    d = dense()
    d.s.dkdv_atomic = 1
    assert status_ws(d)[0] == INVALID
    s = selected()
    s.s.dkdv_atomic = 1
    assert status_ws(s)[0] == UNSUPPORTED
    args = [FAKE] * 8
    n = big
    assert sab.lib.attn_bwd_indexer(_indexer().ref, *args, FAKE, n - 1, None) == WORKSPACE
    a = list(args); a[4] = None
    assert sab.lib.attn_bwd_indexer(_indexer().ref, *a, FAKE, n, None) == NULLPTR
    assert sab.lib.attn_bwd_indexer(selected().ref, *args, FAKE, n, None) == INVALID
