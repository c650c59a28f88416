"""Attention backward (dense varlen FlashAttention-style and NSA selected) on MI355X.

Thin ctypes binding over libattnbwd.so, whose C ABI is declared in
include/attn_bwd.h.  The functions below keep the C names and only marshal
arguments: every step of the backward runs in the library's HIP kernels.  torch
is used for device memory and streams.

    import sparse_attention_backward_amd as sab
    prob = sab.Problem.dense(cu_q, cu_kv, n1, n2, d_qk, d_v, scale, causal=True, d_rope=64)
    dq, dq_rope, dk, dk_rope, dv = sab.dense_backward(prob, q, q_rope, k, k_rope, v, out, dy, smax, ssum)

The library must have been built (``python -m sparse_attention_backward_amd.build``);
importing this package without it raises ImportError -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_int32, c_int64, c_uint64, c_void_p

import torch

__all__ = [
    "AttnError", "Problem", "LIB_PATH", "lib",
    "attn_bwd_workspace_size", "attn_bwd_dense_varlen", "attn_bwd_dense_varlen_noalloc", "attn_bwd_selected",
    "attn_fwd_selected", "attn_bwd_selected_index", "attn_bwd_indexer", "attn_bwd_check_index_flag", "attn_bwd_status_string", "attn_bwd_version",
    "attn_bwd_profiling", "attn_bwd_profile_reset", "attn_bwd_profile_read",
    "dense_backward", "selected_backward", "selected_forward", "indexer_backward", "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattnbwd.so")

ATTN_OK, ATTN_ERR_NULLPTR, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = range(6)
ATTN_BF16, ATTN_FP16, ATTN_FP32 = 0, 1, 2
ATTN_OP_DENSE, ATTN_OP_SELECTED, ATTN_OP_SELECTED_FWD, ATTN_OP_INDEXER = 0, 1, 2, 3
ATTN_LAYOUT_TND, ATTN_LAYOUT_BSND = 0, 1

NOALLOC_SCRATCH_BYTES = 64 << 20  # ATTN_BWD_NOALLOC_SCRATCH_BYTES

EXPORTED_SYMBOLS = ("attn_bwd_workspace_size", "attn_bwd_dense_varlen", "attn_bwd_dense_varlen_noalloc",
                    "attn_bwd_selected", "attn_fwd_selected", "attn_bwd_selected_index", "attn_bwd_indexer",
                    "attn_bwd_check_index_flag", "attn_bwd_profiling", "attn_bwd_profile_reset",
                    "attn_bwd_profile_read", "attn_bwd_status_string", "attn_bwd_version")


class attn_bwd_problem_t(ctypes.Structure):
    _fields_ = [
        ("op", c_int32), ("dtype", c_int32), ("batch", c_int32), ("layout", c_int32),
        ("cu_seqlens_q", POINTER(c_int64)), ("cu_seqlens_kv", POINTER(c_int64)),
        ("seq_len_q", c_int64), ("seq_len_kv", c_int64),
        ("n1", c_int32), ("n2", c_int32),
        ("d_qk", c_int32), ("d_rope", c_int32), ("d_v", c_int32),
        ("scale", c_double), ("causal", c_int32), ("mask_align", c_int32), ("band", c_int32),
        ("pre_tokens", c_int64), ("next_tokens", c_int64),
        ("block_size", c_int32), ("block_count", c_int32),
        ("deterministic", c_int32), ("dkdv_atomic", c_int32), ("dense_dq_mode", c_int32),
        ("sel_window_tokens", c_int32),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_attention_backward_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = POINTER(attn_bwd_problem_t)
    L.attn_bwd_workspace_size.argtypes = [P, POINTER(c_uint64)]
    L.attn_bwd_workspace_size.restype = c_int32
    L.attn_bwd_dense_varlen.argtypes = [P] + [c_void_p] * 7 + [c_void_p, c_void_p] + [c_void_p] * 5 + \
        [c_void_p, c_uint64, c_void_p]
    L.attn_bwd_dense_varlen.restype = c_int32
    L.attn_bwd_dense_varlen_noalloc.argtypes = [P] + [c_void_p] * 7 + [c_void_p, c_void_p] + [c_void_p] * 5 + \
        [c_void_p]
    L.attn_bwd_dense_varlen_noalloc.restype = c_int32
    L.attn_bwd_selected.argtypes = [P] + [c_void_p] * 5 + [c_void_p, c_void_p, c_void_p] + [c_void_p] * 3 + \
        [c_void_p, c_uint64, c_void_p]
    L.attn_bwd_selected.restype = c_int32
    L.attn_fwd_selected.argtypes = [P] + [c_void_p] * 7 + [c_void_p, c_uint64, c_void_p]
    L.attn_fwd_selected.restype = c_int32
    L.attn_bwd_selected_index.argtypes = [P] + [c_void_p] * 4 + [c_void_p, c_uint64, c_void_p]
    L.attn_bwd_selected_index.restype = c_int32
    L.attn_bwd_indexer.argtypes = [P] + [c_void_p] * 8 + [c_void_p, c_uint64, c_void_p]
    L.attn_bwd_indexer.restype = c_int32
    L.attn_bwd_check_index_flag.argtypes = [P, c_void_p, POINTER(c_int32), c_void_p]
    L.attn_bwd_check_index_flag.restype = c_int32
    L.attn_bwd_profiling.argtypes = [c_int32]
    L.attn_bwd_profiling.restype = c_int32
    L.attn_bwd_profile_reset.argtypes = []
    L.attn_bwd_profile_reset.restype = c_int32
    L.attn_bwd_profile_read.argtypes = [c_int32, POINTER(c_char_p), POINTER(c_double), POINTER(c_int64)]
    L.attn_bwd_profile_read.restype = c_int32
    L.attn_bwd_status_string.argtypes = [c_int32]
    L.attn_bwd_status_string.restype = c_char_p
    L.attn_bwd_version.argtypes = []
    L.attn_bwd_version.restype = c_char_p
    return L


_LIB = None


def _L():
    """The loaded library (loaded on first use; ImportError when it is missing)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def __getattr__(name):  # module attribute `lib`, loaded on first access
    if name == "lib":
        return _L()
    raise AttributeError(name)


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__(f"{where}: {_L().attn_bwd_status_string(self.status).decode()} (status {self.status})")


def _check(st, where):
    if st != ATTN_OK:
        raise AttnError(st, where)


class Problem:
    """attn_bwd_problem_t plus the host cu_seqlens arrays it points to (kept alive here)."""

    def __init__(self, op, dtype, cu_q, cu_kv, n1, n2, d_qk, d_v, scale, d_rope=0, causal=False,
                 block_size=0, block_count=0, deterministic=False, dkdv_atomic=False, dense_dq_mode=0,
                 window_tokens=0, bsnd=None, mask_align=0, band=None):
        """bsnd = (B, S1, S2): the BSND layout (cu_q / cu_kv are then ignored and passed as NULL)."""
        if bsnd is not None:
            B, S1, S2 = (int(v) for v in bsnd)
            cu_q = [b * S1 for b in range(B + 1)]
            cu_kv = [b * S2 for b in range(B + 1)]
        cu_q = [int(x) for x in cu_q]
        cu_kv = [int(x) for x in cu_kv]
        self.cu_q_arr = (c_int64 * len(cu_q))(*cu_q)
        self.cu_kv_arr = (c_int64 * len(cu_kv))(*cu_kv)
        null = ctypes.cast(None, POINTER(c_int64))
        self.s = attn_bwd_problem_t(
            op=op, dtype=dtype, batch=len(cu_q) - 1, layout=ATTN_LAYOUT_BSND if bsnd else ATTN_LAYOUT_TND,
            cu_seqlens_q=null if bsnd else ctypes.cast(self.cu_q_arr, POINTER(c_int64)),
            cu_seqlens_kv=null if bsnd else ctypes.cast(self.cu_kv_arr, POINTER(c_int64)),
            seq_len_q=bsnd[1] if bsnd else 0, seq_len_kv=bsnd[2] if bsnd else 0,
            n1=n1, n2=n2, d_qk=d_qk, d_rope=d_rope, d_v=d_v, scale=float(scale), causal=int(bool(causal)),
            mask_align=int(mask_align), band=int(band is not None),
            pre_tokens=int(band[0]) if band is not None else 0, next_tokens=int(band[1]) if band is not None else 0,
            block_size=block_size, block_count=block_count,
            deterministic=int(bool(deterministic)), dkdv_atomic=int(bool(dkdv_atomic)),
            dense_dq_mode=int(dense_dq_mode), sel_window_tokens=int(window_tokens))
        self.T1, self.T2 = cu_q[-1], cu_kv[-1]

    @classmethod
    def dense(cls, cu_q, cu_kv, n1, n2, d_qk, d_v, scale, causal=False, d_rope=0, dtype="bf16",
              deterministic=False, dq_mode=0, align=0, band=None):
        """dq_mode: 0 automatic, 1 stored dS, 2 recompute (field dense_dq_mode of the C struct).
        align: 0 top-left, 1 bottom-right (field mask_align); band = (pre_tokens, next_tokens)."""
        return cls(ATTN_OP_DENSE, {"bf16": ATTN_BF16, "fp32": ATTN_FP32, "fp16": ATTN_FP16}[dtype], cu_q, cu_kv,
                   n1, n2, d_qk, d_v, scale, d_rope=d_rope, causal=causal, deterministic=deterministic,
                   dense_dq_mode=dq_mode, mask_align=align, band=band)

    @classmethod
    def selected(cls, cu_q, cu_kv, n1, n2, d_qk, d_v, scale, block_size, block_count, deterministic=False,
                 dkdv_atomic=False, dtype="bf16", window_tokens=0, forward=False, bsnd=None):
        """window_tokens: query tokens per window (field sel_window_tokens; 0 automatic).
        forward: the problem of attn_fwd_selected (op ATTN_OP_SELECTED_FWD).
        bsnd = (B, S1, S2): BSND layout instead of TND (cu_q / cu_kv ignored)."""
        return cls(ATTN_OP_SELECTED_FWD if forward else ATTN_OP_SELECTED,
                   {"bf16": ATTN_BF16, "fp32": ATTN_FP32, "fp16": ATTN_FP16}[dtype], cu_q,
                   cu_kv, n1, n2, d_qk, d_v, scale, block_size=block_size, block_count=block_count,
                   deterministic=deterministic, dkdv_atomic=dkdv_atomic, window_tokens=window_tokens, bsnd=bsnd)

    @classmethod
    def indexer(cls, cu_q, cu_kv, n1, n2, topk, d=128, deterministic=False, window_tokens=0, bsnd=None,
                dk_atomic=False):
        """The lightning-indexer backward's problem (op ATTN_OP_INDEXER): topk indices per
        (token, key head), head dim d, bf16.  dk_atomic (with deterministic False): dK by fp32
        atomics instead of the ordered sums."""
        return cls(ATTN_OP_INDEXER, ATTN_BF16, cu_q, cu_kv, n1, n2, d, 0, 1.0, block_size=1, block_count=topk,
                   deterministic=deterministic, dkdv_atomic=dk_atomic, window_tokens=window_tokens, bsnd=bsnd)

    @property
    def ref(self):
        return ctypes.byref(self.s)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---- the C functions, same names ----------------------------------------------

def attn_bwd_status_string(status: int) -> str:
    return _L().attn_bwd_status_string(int(status)).decode()


def attn_bwd_version() -> str:
    return _L().attn_bwd_version().decode()


def attn_bwd_workspace_size(problem: Problem) -> int:
    n = c_uint64(0)
    _check(_L().attn_bwd_workspace_size(problem.ref, ctypes.byref(n)), "attn_bwd_workspace_size")
    return int(n.value)


def attn_bwd_dense_varlen(problem, q, q_rope, k, k_rope, v, out, dy, softmax_max, softmax_sum,
                          dq, dq_rope, dk, dk_rope, dv, workspace, workspace_bytes=None, stream=None):
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    st = _L().attn_bwd_dense_varlen(problem.ref, _ptr(q), _ptr(q_rope), _ptr(k), _ptr(k_rope), _ptr(v), _ptr(out),
                                   _ptr(dy), _ptr(softmax_max), _ptr(softmax_sum), _ptr(dq), _ptr(dq_rope), _ptr(dk),
                                   _ptr(dk_rope), _ptr(dv), _ptr(workspace), wb, _stream(stream))
    _check(st, "attn_bwd_dense_varlen")


def attn_bwd_dense_varlen_noalloc(problem, q, q_rope, k, k_rope, v, out, dy, softmax_max, softmax_sum,
                                  dq, dq_rope, dk, dk_rope, dv, stream=None):
    st = _L().attn_bwd_dense_varlen_noalloc(problem.ref, _ptr(q), _ptr(q_rope), _ptr(k), _ptr(k_rope), _ptr(v),
                                           _ptr(out), _ptr(dy), _ptr(softmax_max), _ptr(softmax_sum), _ptr(dq),
                                           _ptr(dq_rope), _ptr(dk), _ptr(dk_rope), _ptr(dv), _stream(stream))
    _check(st, "attn_bwd_dense_varlen_noalloc")


def attn_bwd_selected(problem, q, k, v, out, dy, softmax_max, softmax_sum, topk_indices, dq, dk, dv,
                      workspace, workspace_bytes=None, stream=None):
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    st = _L().attn_bwd_selected(problem.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dy), _ptr(softmax_max),
                               _ptr(softmax_sum), _ptr(topk_indices), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                               wb, _stream(stream))
    _check(st, "attn_bwd_selected")


def attn_fwd_selected(problem, q, k, v, topk_indices, out, softmax_max, softmax_sum, workspace,
                      workspace_bytes=None, stream=None):
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    st = _L().attn_fwd_selected(problem.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(topk_indices), _ptr(out),
                               _ptr(softmax_max), _ptr(softmax_sum), _ptr(workspace), wb, _stream(stream))
    _check(st, "attn_fwd_selected")


def selected_forward(problem, q, k, v, topk_indices, workspace=None, stream=None):
    """Allocate out [T1, N1, d_v] and the [T1, N1, 8] statistics (and the workspace unless given)
    and run attn_fwd_selected.  Returns out, softmax_max, softmax_sum."""
    T1, n1, dv = q.shape[0], q.shape[1], v.shape[-1]
    out = torch.empty((T1, n1, dv), dtype=q.dtype, device=q.device)
    smax = torch.empty((T1, n1, 8), dtype=torch.float32, device=q.device)
    ssum = torch.empty((T1, n1, 8), dtype=torch.float32, device=q.device)
    ws = workspace if workspace is not None else _workspace(problem, q.device)
    attn_fwd_selected(problem, q, k, v, topk_indices, out, smax, ssum, ws, stream=stream)
    return out, smax, ssum


def attn_bwd_selected_index(problem, topk_indices, offsets, lists, order, workspace, workspace_bytes=None,
                            stream=None):
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    st = _L().attn_bwd_selected_index(problem.ref, _ptr(topk_indices), _ptr(offsets), _ptr(lists), _ptr(order),
                                     _ptr(workspace), wb, _stream(stream))
    _check(st, "attn_bwd_selected_index")


def attn_bwd_indexer(problem, q, k, weights, dy, indices, dq, dk, dweights, workspace, workspace_bytes=None,
                     stream=None):
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    st = _L().attn_bwd_indexer(problem.ref, _ptr(q), _ptr(k), _ptr(weights), _ptr(dy), _ptr(indices), _ptr(dq),
                              _ptr(dk), _ptr(dweights), _ptr(workspace), wb, _stream(stream))
    _check(st, "attn_bwd_indexer")


def indexer_backward(problem, q, k, weights, dy, indices, workspace=None, stream=None):
    """Allocate dq, dk, dweights (and the workspace unless given) and run attn_bwd_indexer."""
    dq, dk, dw = torch.empty_like(q), torch.empty_like(k), torch.empty_like(weights)
    ws = workspace if workspace is not None else _workspace(problem, q.device)
    attn_bwd_indexer(problem, q, k, weights, dy, indices, dq, dk, dw, ws, stream=stream)
    return dq, dk, dw


def attn_bwd_check_index_flag(problem, workspace, stream=None) -> bool:
    r = c_int32(0)
    _check(_L().attn_bwd_check_index_flag(problem.ref, _ptr(workspace), ctypes.byref(r), _stream(stream)),
           "attn_bwd_check_index_flag")
    return bool(r.value)


def attn_bwd_profiling(enable: bool) -> None:
    _check(_L().attn_bwd_profiling(int(bool(enable))), "attn_bwd_profiling")


def attn_bwd_profile_reset() -> None:
    _check(_L().attn_bwd_profile_reset(), "attn_bwd_profile_reset")


def attn_bwd_profile_read() -> dict:
    """All per-kernel totals: {name: (total_ms, launches)} (synchronises on the events)."""
    out, i = {}, 0
    while True:
        name, ms, n = c_char_p(), c_double(), c_int64()
        st = _L().attn_bwd_profile_read(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(n))
        if st == ATTN_ERR_INVALID:
            return out
        _check(st, "attn_bwd_profile_read")
        out[name.value.decode()] = (ms.value, n.value)
        i += 1


# ---- allocation helpers (torch owns the memory) ----------------------------------

def _workspace(problem, device):
    n = attn_bwd_workspace_size(problem)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def dense_backward(problem, q, q_rope, k, k_rope, v, out, dy, softmax_max, softmax_sum, workspace=None,
                   stream=None):
    """Allocate outputs (and the workspace unless given) and run attn_bwd_dense_varlen.
    Returns dq, dq_rope, dk, dk_rope, dv (rope outputs are None without rope)."""
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dq_rope = torch.empty_like(q_rope) if q_rope is not None else None
    dk_rope = torch.empty_like(k_rope) if k_rope is not None else None
    ws = workspace if workspace is not None else _workspace(problem, q.device)
    attn_bwd_dense_varlen(problem, q, q_rope, k, k_rope, v, out, dy, softmax_max, softmax_sum,
                          dq, dq_rope, dk, dk_rope, dv, ws, stream=stream)
    return dq, dq_rope, dk, dk_rope, dv


def selected_backward(problem, q, k, v, out, dy, softmax_max, softmax_sum, topk_indices, workspace=None,
                      stream=None):
    """Allocate outputs (and the workspace unless given) and run attn_bwd_selected.
    Returns dq, dk, dv."""
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = workspace if workspace is not None else _workspace(problem, q.device)
    attn_bwd_selected(problem, q, k, v, out, dy, softmax_max, softmax_sum, topk_indices, dq, dk, dv, ws,
                      stream=stream)
    return dq, dk, dv
