"""GPU parity on seeded random problems: selected backward (with and without attentionOut,
windows, determinism settings, bf16 / fp16, uniform / Zipf ids), selected forward, dense (bf16
and fp32, causal aligned either way, windows, no mask, the three dQ modes) and the indexer
backward in its three modes, each against the float64 oracle at the stated tolerances.
Shapes are drawn per case from a seed: ragged and empty sequences, block sizes 16..128,
G from 1 to 64, head dims 128 / 192."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_backward_amd as sab
import workloads as W
from helpers import assert_close, check_against_oracle, f64, gpu_backward, oracle_backward, oracle_forward

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("i", range(40))
def test_random_problem(i):
    seed = 20000 + i
    rng = np.random.default_rng(seed)
    kind = ["selected", "selected", "dense", "forward", "indexer"][i % 5]
    if kind in ("selected", "forward"):
        bs = int(rng.choice([16, 32, 48, 64, 80, 96, 112, 128]))
        n2 = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 3, 5, 8, 12, 16, 20, 32]))
        cnt = int(rng.integers(1, 6))
        nseq = int(rng.integers(1, 4))
        lq = tuple(int(x) for x in rng.integers(0, 90, nseq))
        if sum(lq) == 0:
            lq = (17,) + lq[1:]
        lk = tuple(int(bs * rng.integers(cnt, cnt + 4)) for _ in range(nseq))
        d_qk = int(rng.choice([128, 192]))
        dtype = str(rng.choice(["bf16", "fp16"]))
        dist = str(rng.choice(["uniform", "zipf"]))
        w = W.small_selected(seqlens=lq, seqlens_kv=lk, n1=G * n2, n2=n2, d_qk=d_qk, block_size=bs,
                             block_count=cnt, index_dist=dist, seed=seed, dtype=dtype)
        desc = f"{kind} lq={lq} lk={lk} G={G} n2={n2} bs={bs} cnt={cnt} dqk={d_qk} {dtype} {dist}"
        x = W.make_inputs(w)
        if kind == "selected":
            with_out = bool(rng.integers(0, 2))
            wt = int(rng.choice([0, 0, 7, 31]))
            det = bool(rng.integers(0, 2))
            desc += f" out={with_out} win={wt} det={det}"
            print("[random]", i, desc, flush=True)
            o, smax, ssum = oracle_forward(w, x)
            got = gpu_backward(w, x, o if with_out else None, smax, ssum, deterministic=det, window_tokens=wt)
            check_against_oracle(w, got, oracle_backward(w, x))
        else:
            wt = int(rng.choice([0, 0, 9, 40]))
            desc += f" win={wt}"
            print("[random]", i, desc, flush=True)
            dev = torch.device("cuda", 0)
            g = lambda t: t.to(dev).contiguous()  # noqa: E731
            fw = sab.Problem.selected(w.cu_q, w.cu_kv, w.n1, w.n2, w.d_qk, w.d_v, w.scale, w.block_size,
                                      w.block_count, dtype=w.dtype, forward=True, window_tokens=wt)
            out, smax, ssum = sab.selected_forward(fw, g(x["query"]), g(x["key"]), g(x["value"]), g(x["topk"]))
            torch.cuda.synchronize()
            o, m, l = O.forward_selected(f64(x["query"]), f64(x["key"]), f64(x["value"]), x["topk"].numpy(),
                                         w.cu_q, w.cu_kv, w.n1, w.n2, w.scale, w.block_size)
            assert_close("out", f64(out), o, w.dtype)
            sm = f64(smax)[..., 0]
            ss = f64(ssum)[..., 0]
            assert np.all(np.abs(sm - m) <= 1e-3 * np.maximum(1, np.abs(m))), "smax"
            assert np.all(np.abs(ss - l) <= 1e-3 * np.abs(l) + 1e-30), "ssum"
    elif kind == "dense":
        n2 = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 4, 8]))
        nseq = int(rng.integers(1, 4))
        lq = tuple(int(x) for x in rng.integers(0, 200, nseq))
        if sum(lq) == 0:
            lq = (33,) + lq[1:]
        mode = str(rng.choice(["causal", "causal_br", "band", "none"]))
        if mode in ("causal_br", "band", "none"):
            lk = tuple(int(x) for x in rng.integers(0, 220, nseq))
        else:
            lk = lq
        dims = [(128, 64, 128), (128, 0, 128), (64, 0, 64)][int(rng.integers(0, 3))]
        dtype = str(rng.choice(["bf16", "bf16", "fp32"]))
        if dtype == "fp32":
            dims = (64, 0, 64)
        band = None
        causal = mode in ("causal", "causal_br")
        align = 1 if mode == "causal_br" else int(rng.integers(0, 2))
        if mode == "band":
            band = (int(rng.integers(-5, 60)), int(rng.integers(-5, 60)))
            if band[0] + band[1] < 0:
                band = (band[0], -band[0])
        if mode == "none":
            align = 0
        w = W.small_dense(seqlens=lq, seqlens_kv=lk, n1=G * n2, n2=n2, d_qk=dims[0], d_rope=dims[1],
                          d_v=dims[2], dtype=dtype, causal=causal, seed=seed, mask_align=align, band=band)
        dq_mode = int(rng.choice([0, 1, 2])) if dtype == "bf16" else 0
        desc = (f"dense lq={lq} lk={lk} G={G} n2={n2} dims={dims} {dtype} mode={mode} align={align} band={band} "
                f"dq={dq_mode}")
        print("[random]", i, desc, flush=True)
        x = W.make_inputs(w)
        o, smax, ssum = oracle_forward(w, x)
        got = gpu_backward(w, x, o, smax, ssum, dq_mode=dq_mode)
        check_against_oracle(w, got, oracle_backward(w, x))
    else:
        n2 = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 5, 16, 24, 32, 64]))
        nseq = int(rng.integers(1, 3))
        lq = tuple(int(x) for x in rng.integers(1, 60, nseq))
        topk = int(rng.integers(1, 150))
        lk = tuple(int(x) + topk for x in rng.integers(0, 100, nseq))
        mode = str(rng.choice(["ordered", "det", "atomic"]))
        wt = int(rng.choice([0, 0, 11]))
        w = W.small_indexer(seqlens=lq, seqlens_kv=lk, n1=G * n2, n2=n2, topk=topk, seed=seed)
        desc = f"indexer lq={lq} lk={lk} G={G} n2={n2} topk={topk} mode={mode} win={wt}"
        print("[random]", i, desc, flush=True)
        x = W.make_indexer_inputs(w)
        q64, k64, idx = f64(x["q"]), f64(x["k"]), x["indices"].numpy()
        seq = np.searchsorted(w.cu_q, np.arange(w.T1), side="right") - 1
        # scores within 1e-3 of zero get dy = 0: the ReLU decision (fp32 here, float64 in the
        # oracle) then cannot change an entry's contribution
        dy = x["dy"].clone()
        for t in range(w.T1):
            for h in range(w.n2):
                rows = w.cu_kv[seq[t]] + idx[t, h].astype(np.int64)
                S = q64[t, h * w.G:(h + 1) * w.G] @ k64[rows, h].T
                dy[t, h, torch.from_numpy((np.abs(S) < 1e-3).any(axis=0))] = 0
        x["dy"] = dy
        dev = torch.device("cuda", 0)
        g = lambda t: t.to(dev).contiguous()  # noqa: E731
        prob = sab.Problem.indexer(w.cu_q, w.cu_kv, w.n1, w.n2, w.topk, deterministic=mode == "det",
                                   window_tokens=wt, dk_atomic=mode == "atomic")
        dq, dk, dw = sab.indexer_backward(prob, g(x["q"]), g(x["k"]), g(x["weights"]), g(x["dy"]), g(x["indices"]))
        torch.cuda.synchronize()
        rq, rk, rw = O.indexer_backward(q64, k64, f64(x["weights"]), f64(x["dy"]), idx, w.cu_q, w.cu_kv,
                                        w.n1, w.n2)
        assert_close("dq", f64(dq), rq, "bf16")
        assert_close("dk", f64(dk), rk, "bf16")
        assert_close("dw", f64(dw), rw, "bf16")
