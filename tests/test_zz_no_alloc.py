"""attn_bwd_dense_varlen_noalloc: the dense backward with the library's fixed scratch array
instead of a caller workspace.  Called through the C ABI and compared with
attn_bwd_dense_varlen on the same inputs (same dQ mode: bitwise equal, the same kernels run
on the same plan) and with the float64 oracle (bf16 / fp32 tolerances), on calls in a row
whose later problems are smaller, so that stale scratch contents would show."""
import pytest
import torch

import sparse_attention_backward_amd as sab
import workloads as W
from helpers import check_against_oracle, oracle_backward, oracle_forward, problem_for

pytestmark = pytest.mark.gpu


def _outs(x, dev):
    e = lambda t: None if t is None else torch.empty_like(t, device=dev)  # noqa: E731
    return [e(x["query"]), e(x["query_rope"]), e(x["key"]), e(x["key_rope"]), e(x["value"])]


def _call_both(w, dq_mode):
    dev = torch.device("cuda", 0)
    x = W.make_inputs(w)
    o, smax, ssum = oracle_forward(w, x)
    g = lambda t: None if t is None else t.to(dev).contiguous()  # noqa: E731
    args = (g(x["query"]), g(x["query_rope"]), g(x["key"]), g(x["key_rope"]), g(x["value"]), g(o), g(x["dy"]),
            g(smax), g(ssum))
    prob = problem_for(w, dq_mode=dq_mode)
    print(f"[noalloc] {w.name} seqlens={w.seqlens_q} n1={w.n1} n2={w.n2} dq_mode={dq_mode} "
          f"workspace={sab.attn_bwd_workspace_size(prob)}", flush=True)
    a = _outs(x, dev)
    sab.attn_bwd_dense_varlen_noalloc(prob, *args, *a)
    torch.cuda.synchronize()
    b = _outs(x, dev)
    ws = torch.empty(max(1, sab.attn_bwd_workspace_size(prob)), dtype=torch.uint8, device=dev)
    sab.attn_bwd_dense_varlen(prob, *args, *b, ws)
    torch.cuda.synchronize()
    names = ("dq", "dq_rope", "dk", "dk_rope", "dv")
    for n, ta, tb in zip(names, a, b):
        if ta is not None:
            assert torch.equal(ta, tb), f"{w.name}:{n}: no-alloc result differs from the workspace call"
    check_against_oracle(w, dict(zip(names, a)), oracle_backward(w, x))


def test_noalloc_matches_workspace_call_calls_in_a_row():
    # larger first, then smaller problems on the same scratch array
    _call_both(W.small_dense(seqlens=(300, 130), n1=8, n2=2), dq_mode=0)
    _call_both(W.small_dense(seqlens=(97,), n1=4, n2=1, d_qk=64, d_rope=0, d_v=64), dq_mode=0)
    _call_both(W.small_dense(seqlens=(190,), n1=6, n2=3), dq_mode=2)
    _call_both(W.small_dense(seqlens=(70,), n1=2, n2=2), dq_mode=2)
    _call_both(W.config(1), dq_mode=0)   # fp32


def test_noalloc_refuses_problems_beyond_the_scratch_array():
    w = W.small_dense(seqlens=(300000,), n1=32, n2=8)   # row statistics alone exceed 64 MiB
    prob = problem_for(w, dq_mode=2)
    assert sab.attn_bwd_workspace_size(prob) > sab.NOALLOC_SCRATCH_BYTES
    fake = 0x10000  # never dereferenced: the call returns before enqueueing anything
    with pytest.raises(sab.AttnError) as e:
        sab.attn_bwd_dense_varlen_noalloc(prob, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                          fake, fake, fake)
    assert e.value.status == sab.ATTN_ERR_WORKSPACE
