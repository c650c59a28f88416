// Dense KV-major backward: dK and dV accumulated in registers, plus the dS tiles that
// the dQ product consumes (bf16 MFMA, fp32 accumulation).
//
// Page "aclnnFlashAttentionUnpaddingScoreGradV3", Formula section: dV = P^T dY,
// dK = dS^T Q / sqrt(d), dkRope = dS^T qRope / sqrt(d), with Q = [query, queryRope].
//
// One workgroup (4 waves) owns a 64-key tile of one sequence and KV head.  Query rows
// stream past in steps of 64 rows: for each of the G query heads of the KV head, the
// query tiles from the last one down to the diagonal (causal) or down to the first.
// Walking every key tile's list from the same end keeps the workgroups of one
// (sequence, KV head) on the same query tile at the same time, so their row loads
// share the L2.
//
// The waves form a 2 x 2 grid: wave w owns keys 32(w&1) .. +31 of the tile (K and V
// resident in registers as MFMA B operands) and rows 32(w>>1) .. +31 of every step.
// Per step and wave (32 rows x 32 keys):
//   S = Q K^T, dP = dY V^T       A operands: Q / dY rows from LDS (16-byte reads)
//   P = exp2(S*scale*log2e - lse2), dS = P (dP - drow)   (masks: causal diagonal,
//                                 ragged query tail, ragged key tail)
//   dV += P^T dY, dK += dS^T Q   A operands: the P / dS C tiles repacked in registers;
//                                 B operands: dY / Q columns (ds_read_b64_tr_b16)
//   dS^T -> workspace (bf16), one 64 x 64 block per (query tile, key tile, head)
// Each key row's dK / dV is the sum of the two row-half waves' registers, added once
// through LDS at the end.  Every output row has one writer: no atomics, deterministic.
//
// Staging: a step's Q / dY / lse2 / drow land in one of three LDS stages, moved by
// global->LDS transfers issued two steps ahead.  Stage tiles are chunk-major: the
// 16-byte chunk c of row r sits at byte c * kCB + 16 r, so one transfer moves one chunk
// of all 64 rows (lane = row) and every LDS read is a per-lane base plus an immediate.
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

constexpr int kRows = 64;        // query rows per step, keys per workgroup
constexpr int kCB = 1024 + 128;  // bytes per chunk column of a staged 64-row tile
typedef __attribute__((address_space(3))) void lds_void;

struct DkvArgs {
  const uint16_t* q; const uint16_t* q_rope;
  const uint16_t* k; const uint16_t* k_rope;
  const uint16_t* v; const uint16_t* dy;
  const float* lse2; const float* drow;
  uint16_t* dk; uint16_t* dk_rope; uint16_t* dv;
  uint16_t* ds;               // [block][head][64 keys][64 rows] bf16 (dS transposed)
  const int64_t* cu_q; const int64_t* cu_kv;
  const int64_t* ds_base;     // [B + 1] (query tile, key tile) blocks before each sequence
  const int32_t* tiles;       // [n][3] (sequence, key tile, KV head); sequence < 0: idle slot
  int n1, n2, G, d_main, d_rope, d_v;
  int causal;
  float scale, scale_log2e;
};

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that keeps the compiler from moving memory accesses across it but,
// unlike __syncthreads(), does not wait for this wave's outstanding global->LDS
// transfers and stores.  Each wave first waits for the transfers it needs.
__device__ __forceinline__ void barrier_no_vm_wait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* lds) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds);
}
// global -> LDS transfer of 16 bytes per lane: lane l reads `src` + OFF and writes LDS
// byte M0 + OFF + 16 l with M0 = `lds` + MOFF.  Inline assembly keeps the compiler from
// adding waits of its own: every wait on these transfers is an explicit wait_vmcnt.
template <int MOFF, int OFF>
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%3"
               ::"v"(src), "s"(lds), "i"(MOFF), "i"(OFF) : "memory", "m0", "scc");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
// 8-byte store issued as inline assembly as well, so that the compiler does not insert a
// full vmcnt wait before the next step's transfers (it cannot see that the waits on
// those transfers are exact; see the ordering note in the step loop).
__device__ __forceinline__ void st8(void* dst, i16x4 v) {
  asm volatile("global_store_dwordx2 %0, %1, off" ::"v"(dst), "v"(v) : "memory");
}

template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

template <typename T>
__device__ __forceinline__ const T* at_bytes(const void* base, int bytes) {
  return reinterpret_cast<const T*>(static_cast<const char*>(base) + bytes);
}

template <int DQK, int DV, bool DS>
__global__ __launch_bounds__(256, 1) void dense_kv_kernel(DkvArgs a) {
  constexpr int KS = DQK / 32, VS = DV / 32, NQ = DQK / 16, NV = DV / 16;
  constexpr int QCH = DQK / 8, YCH = DV / 8;   // 16-byte chunks per row
  constexpr int QLD = QCH / 4, YLD = YCH / 4;  // transfer instructions per wave per tile
  constexpr int NLD = QLD + YLD + 2;           // + lse2, drow
  constexpr int QB = QCH * kCB, YB = YCH * kCB;
  constexpr int SB = QB + YB + 2 * 256;        // one stage: Q, dY, lse2, drow
  static_assert(3 * SB <= 160 * 1024, "three stages must fit in LDS");
  static_assert(2 * 2 * (NQ + NV) * 1024 + (QCH + YCH) * kCB <= 3 * SB, "epilogue buffers must fit");
  __shared__ __attribute__((aligned(16))) char smem[3 * SB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = w & 1, rh = w >> 1;
  const int l16 = lane & 15, g = lane >> 4, jj = l16 >> 2, qq = l16 & 3;

  const int b = a.tiles[3 * blockIdx.x];
  if (b < 0) return;  // idle slot of the schedule
  const int kt0 = a.tiles[3 * blockIdx.x + 1];
  const int kvh = a.tiles[3 * blockIdx.x + 2];
  const int64_t ks = a.cu_kv[b];
  const int S2 = (int)(a.cu_kv[b + 1] - ks);
  const int64_t k0 = ks + (int64_t)kt0 * kRows;
  const int nk = min(kRows, S2 - kt0 * kRows);
  const int nkt = (S2 + kRows - 1) / kRows;
  const int64_t qs = a.cu_q[b];
  const int S1 = (int)(a.cu_q[b + 1] - qs);
  const int nqt = (S1 + kRows - 1) / kRows;
  const int qt0 = a.causal ? min(kt0, nqt) : 0;
  const int nq = nqt - qt0;
  const int nsteps = a.G * nq;
  const int qmain = a.d_main / 8;  // chunks of a Q row that come from `query` (the rest: queryRope)
  const int64_t blk0 = a.ds_base[b];

  // ---- resident keys: K and V as MFMA B operands ------------------------------------
  bf16x8 Kf[2][KS], Vf[2][VS];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = 32 * kh + 16 * t + l16;
    const bool valid = key < nk;
    const int64_t kr = (k0 + key) * a.n2 + kvh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int d = 32 * s + 8 * g;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (valid) x = ldg16(d < a.d_main ? a.k + kr * a.d_main + d : a.k_rope + kr * a.d_rope + (d - a.d_main));
      Kf[t][s] = __builtin_bit_cast(bf16x8, x);
    }
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (valid) x = ldg16(a.v + kr * a.d_v + 32 * s + 8 * g);
      Vf[t][s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x4 dK[2][NQ], dV[2][NV];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) dK[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NV; ++n) dV[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Per-lane LDS byte offsets within a stage.  Row reads: rows 32rh + 16rt + l16, chunk
  // 4s + g.  Column reads: rows 32rh + 4g + jj (+16), chunk 2j + qq/2, half qq&1.
  const int rd_row = g * kCB + 16 * (32 * rh + l16);
  const int rd_col = (qq >> 1) * kCB + 16 * (32 * rh + 4 * g + jj) + 8 * (qq & 1);

  // step st -> (head hg, query tile qt), query tiles walked from the last one down
  auto step_tile = [&](int st, int& hg, int& qt) {
    hg = st / nq;
    qt = nqt - 1 - (st - hg * nq);
  };

  // issue(): wave w moves chunks c = w + 4k of the 64 rows (lane = row) into one stage.
  // Chunk c lands at c * kCB in the stage: with the per-lane row address + 16 w and the
  // stage + w * kCB as bases, chunk k is the immediate 64 k (global) / 4 k kCB (LDS).
  const int kq = (qmain - w + 3) >> 2;  // chunks k < kq come from `query`, the rest from queryRope
  const uint32_t smem_lds = lds_addr(smem);
  auto issue = [&](int st, int soff) {
    int hg, qt;
    step_tile(st, hg, qt);
    const int h = kvh * a.G + hg;
    const int nvalid = min(kRows, S1 - qt * kRows);
    const int64_t r0 = qs + (int64_t)qt * kRows;
    const int64_t qr = (r0 + min(lane, nvalid - 1)) * a.n1 + h;
    const char* qrow = reinterpret_cast<const char*>(a.q + qr * a.d_main) + 16 * w;
    const char* rrow = reinterpret_cast<const char*>(a.q_rope + qr * a.d_rope) + 16 * (w - qmain);
    const char* yrow = reinterpret_cast<const char*>(a.dy + qr * a.d_v) + 16 * w;
    const uint32_t qb = smem_lds + soff + w * kCB, yb = smem_lds + soff + QB + w * kCB;
    static_for<QLD>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      dma16<k * (4 * kCB - 64), 64 * k>(k < kq ? qrow : rrow, qb);
    });
    static_for<YLD>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      dma16<k * (4 * kCB - 64), 64 * k>(yrow, yb);
    });
    // lse2 / drow of rows 16w .. 16w+15 (lanes 0..15)
    const int64_t lr = (r0 + min(16 * w + l16, nvalid - 1)) * a.n1 + h;
    if (lane < 16) dma4(a.lse2 + lr, smem_lds + soff + QB + YB + 64 * w);
    if (lane < 16) dma4(a.drow + lr, smem_lds + soff + QB + YB + 256 + 64 * w);
  };

  // dS of the previous step, stored at the start of the next one (see the loop)
  i16x4 dsv[2][2];
  uint16_t* dsp = nullptr;

  auto step = [&](int st, const char* stage) {
    int hg, qt;
    step_tile(st, hg, qt);
    const int h = kvh * a.G + hg;
    const int nvalid = min(kRows, S1 - qt * kRows);
    const bool diag = a.causal && qt == kt0;
    // the block's dS^T: [64 keys][64 rows] of (query tile qt, key tile kt0, head h)
    if constexpr (DS) {
      const int64_t blk = blk0 + (a.causal ? (int64_t)qt * (qt + 1) / 2 + kt0 : (int64_t)qt * nkt + kt0);
      dsp = a.ds + (blk * a.n1 + h) * (int64_t)(kRows * kRows) + (32 * kh + l16) * kRows + 32 * rh + 4 * g;
    }
    if (diag && kh > rh) {  // every key of this wave lies after every row: P = dS = 0
#pragma unroll
      for (int t = 0; t < 2; ++t) dsv[t][0] = dsv[t][1] = i16x4{0, 0, 0, 0};
      return;
    }
    const char* Qs = stage;
    const char* Ys = stage + QB;
    const float* Ls = at_bytes<float>(stage, QB + YB);
    const float* Rs = at_bytes<float>(stage, QB + YB + 256);

    // S = Q K^T, dP = dY V^T for both key tiles; the A fragments are shared by them
    bf16x8 qa[2][KS], ya[2][VS];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int s = 0; s < KS; ++s) qa[rt][s] = *at_bytes<bf16x8>(Qs, rd_row + 4 * s * kCB + 256 * rt);
#pragma unroll
      for (int s = 0; s < VS; ++s) ya[rt][s] = *at_bytes<bf16x8>(Ys, rd_row + 4 * s * kCB + 256 * rt);
    }
    f32x4 S[2][2], D[2][2];  // [key tile][row tile]
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        S[t][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        D[t][rt] = S[t][rt];
#pragma unroll
        for (int s = 0; s < KS; ++s) S[t][rt] = mfma_16x16x32(qa[rt][s], Kf[t][s], S[t][rt]);
#pragma unroll
        for (int s = 0; s < VS; ++s) D[t][rt] = mfma_16x16x32(ya[rt][s], Vf[t][s], D[t][rt]);
      }
    // P and dS in place
    f32x4 lse[2], dr[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      lse[rt] = *reinterpret_cast<const f32x4*>(&Ls[32 * rh + 16 * rt + 4 * g]);
      dr[rt] = *reinterpret_cast<const f32x4*>(&Rs[32 * rh + 16 * rt + 4 * g]);
    }
    const bool masked = diag || nvalid < kRows || nk < kRows;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = 32 * kh + 16 * t + l16;  // local to the key tile
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = __builtin_amdgcn_exp2f(S[t][rt][i] * a.scale_log2e - lse[rt][i]);
          if (masked) {
            const int r = 32 * rh + 16 * rt + 4 * g + i;  // local to the query tile
            const bool off = r >= nvalid || key >= nk || (diag && key > r);
            p = off ? 0.f : p;
          }
          D[t][rt][i] = p * (D[t][rt][i] - dr[rt][i]);
          S[t][rt][i] = p;
        }
    }
    // dV += P^T dY, dK += dS^T Q; the column fragments are shared by both key tiles
    bf16x8 pa[2], da[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      pa[t] = pack8(S[t][0], S[t][1]);
      da[t] = pack8(D[t][0], D[t][1]);
      dsv[t][0] = pack4(D[t][0]);
      dsv[t][1] = pack4(D[t][1]);
    }
    auto colfrag = [&](const char* base, int j) -> bf16x8 {
      const int o = rd_col + 2 * j * kCB;
      return join8(lds_read_tr16(reinterpret_cast<const uint16_t*>(base + o)),
                   lds_read_tr16(reinterpret_cast<const uint16_t*>(base + o + 256)));
    };
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const bf16x8 bv = colfrag(Ys, j);
      dV[0][j] = mfma_16x16x32(pa[0], bv, dV[0][j]);
      dV[1][j] = mfma_16x16x32(pa[1], bv, dV[1][j]);
    }
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const bf16x8 bq = colfrag(Qs, j);
      dK[0][j] = mfma_16x16x32(da[0], bq, dK[0][j]);
      dK[1][j] = mfma_16x16x32(da[1], bq, dK[1][j]);
    }
  };

  auto store_ds = [&]() {
    // rows 32rh + 4g + (0..3) and + 16; keys 32kh + 16t + l16
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st8(dsp + 16 * t * kRows, dsv[t][0]);
      st8(dsp + 16 * t * kRows + 16, dsv[t][1]);
    }
  };

  // Ordering of the vector-memory operations.  Iteration st: wait for stage st, barrier,
  // store the dS of step st-1, issue the transfers of stage st+2, compute step st.  At
  // the top of iteration st the operations issued after stage st's transfers are the
  // stores of step st-2 and the transfers of stage st+1, in that order.  Loads complete
  // in order, so "at most NLD outstanding" can only hold once stage st has landed,
  // however the stores complete.
  if (nsteps > 0) issue(0, 0);
  if (nsteps > 1) issue(1, SB);
  for (int st = 0; st < nsteps; ++st) {
    if (st + 1 < nsteps) wait_vmcnt<NLD>();
    else wait_vmcnt<0>();
    barrier_no_vm_wait();  // every wave's share of stage st is in LDS; stage st-1 is free
    if (DS && st > 0) store_ds();
    const int ph = st % 3;
    if (st + 2 < nsteps) issue(st + 2, (ph == 0 ? 2 : ph - 1) * SB);
    step(st, smem + ph * SB);
  }
  if (DS && nsteps > 0) store_ds();

  // ---- epilogue: sum the two row halves, bf16 through LDS, 16-byte stores ------------
  __syncthreads();
  // partials of the rh = 1 waves: [kh][index][lane] as f32x4 (conflict-free)
  f32x4* part = reinterpret_cast<f32x4*>(smem);
  constexpr int NACC = 2 * (NQ + NV);
  if (rh == 1) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int n = 0; n < NQ; ++n) part[(kh * NACC + t * (NQ + NV) + n) * 64 + lane] = dK[t][n];
#pragma unroll
      for (int n = 0; n < NV; ++n) part[(kh * NACC + t * (NQ + NV) + NQ + n) * 64 + lane] = dV[t][n];
    }
  }
  __syncthreads();
  char* outt = smem + 2 * NACC * 1024;  // [chunk][64 keys] output tile, chunk-major
  uint16_t* Ko = reinterpret_cast<uint16_t*>(outt);
  uint16_t* Vo = reinterpret_cast<uint16_t*>(outt + QCH * kCB);
  if (rh == 0) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        const f32x4 o = part[(kh * NACC + t * (NQ + NV) + n) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 32 * kh + 16 * t + 4 * g + i, col = 16 * n + l16;
          Ko[((col >> 3) * kCB + 16 * r) / 2 + (col & 7)] = f2bf((dK[t][n][i] + o[i]) * a.scale);
        }
      }
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        const f32x4 o = part[(kh * NACC + t * (NQ + NV) + NQ + n) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 32 * kh + 16 * t + 4 * g + i, col = 16 * n + l16;
          Vo[((col >> 3) * kCB + 16 * r) / 2 + (col & 7)] = f2bf(dV[t][n][i] + o[i]);
        }
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < kRows * QCH; idx += 256) {
    const int r = idx / QCH, c = idx - r * QCH, d = 8 * c;
    if (r < nk) {
      const int64_t kr = (k0 + r) * a.n2 + kvh;
      uint16_t* dst = d < a.d_main ? a.dk + kr * a.d_main + d : a.dk_rope + kr * a.d_rope + (d - a.d_main);
      sts16(dst, *at_bytes<uint4>(outt, c * kCB + 16 * r));
    }
  }
  for (int idx = tid; idx < kRows * YCH; idx += 256) {
    const int r = idx / YCH, c = idx - r * YCH;
    if (r < nk)
      sts16(a.dv + ((k0 + r) * a.n2 + kvh) * a.d_v + 8 * c, *at_bytes<uint4>(outt, QCH * kCB + c * kCB + 16 * r));
  }
}

}  // namespace

bool dense_bf16_supported(int d_qk_total, int d_v) {
  return (d_qk_total == 192 && d_v == 128) || (d_qk_total == 128 && d_v == 128) || (d_qk_total == 64 && d_v == 64);
}

hipError_t launch_dense_kv_bf16(const DenseArgs& a, hipStream_t s) {
  if (a.n_kv_tiles == 0) return hipSuccess;
  DkvArgs k{};
  k.q = (const uint16_t*)a.q; k.q_rope = (const uint16_t*)a.q_rope;
  k.k = (const uint16_t*)a.k; k.k_rope = (const uint16_t*)a.k_rope;
  k.v = (const uint16_t*)a.v; k.dy = (const uint16_t*)a.dy;
  k.lse2 = a.lse2; k.drow = a.drow;
  k.dk = (uint16_t*)a.dk; k.dk_rope = (uint16_t*)a.dk_rope; k.dv = (uint16_t*)a.dv;
  k.ds = (uint16_t*)a.ds;
  k.cu_q = a.cu_q; k.cu_kv = a.cu_kv; k.ds_base = a.ds_base; k.tiles = a.kv_tiles;
  k.n1 = a.n1; k.n2 = a.n2; k.G = a.G;
  k.d_main = a.d_main; k.d_rope = a.d_rope; k.d_v = a.d_v;
  k.causal = a.causal; k.scale = a.scale; k.scale_log2e = a.scale_log2e;
  const dim3 grid(a.n_kv_tiles);
  const int dqk = a.d_main + a.d_rope;
  const bool ds = a.ds != nullptr;
#define ATTN_KV_LAUNCH(DQ, DV_)                                                                      \
  if (ds) hipLaunchKernelGGL((dense_kv_kernel<DQ, DV_, true>), grid, dim3(256), 0, s, k);            \
  else hipLaunchKernelGGL((dense_kv_kernel<DQ, DV_, false>), grid, dim3(256), 0, s, k);
  if (dqk == 192 && a.d_v == 128) { ATTN_KV_LAUNCH(192, 128) }
  else if (dqk == 128 && a.d_v == 128) { ATTN_KV_LAUNCH(128, 128) }
  else if (dqk == 64 && a.d_v == 64) { ATTN_KV_LAUNCH(64, 64) }
  else return hipErrorInvalidValue;
#undef ATTN_KV_LAUNCH
  return hipGetLastError();
}

}  // namespace ab
