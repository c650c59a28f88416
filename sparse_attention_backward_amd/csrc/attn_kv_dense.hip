// Dense KV-major backward: dK, dV (bf16 MFMA, fp32 accumulation in registers).
//
// Page "aclnnFlashAttentionUnpaddingScoreGradV3", Formula section: dV = P^T dY,
// dK = dS^T Q / sqrt(d), dkRope = dS^T qRope / sqrt(d), with Q = [query, queryRope].
//
// One workgroup (4 waves) owns a 64-row key tile of one sequence and KV head.  Wave w
// holds keys 16w..16w+15: K as MFMA B operands in registers, V in LDS.  Query rows stream
// past in steps of 64 rows (each of the G query heads of the KV head, query tiles from
// the diagonal on when causal).  Per step: S = Q K^T and dP = dY V^T (A operands from
// LDS), P = exp2(S*scale*log2e - lse2) with the causal / ragged-tail mask, dS = P (dP - drow),
// then dV += P^T dY and dK += dS^T Q with the P / dS C tiles reused as A operands and
// dY / Q read column-wise with ds_read_b64_tr_b16.
//
// LDS tiles are chunk-major: the 16-byte chunk c of row r (r < 64) sits at byte
// c * CB + 16 r.  A global->LDS transfer (global_load_lds_dwordx4) then moves one chunk of
// all 64 rows -- lane = row -- into 1 KB of contiguous LDS, and every LDS read is a
// per-lane base plus a compile-time offset.  A 16-row read of one chunk covers 256
// contiguous bytes (all 64 banks); CB = 1024 + 128 puts the two chunks of a column read
// 32 banks apart, so the transposed reads are conflict free as well.
//
// Each step's Q / dY / lse2 / drow tiles go to one of three LDS stages two steps ahead of
// their use, so their load latency hides behind two steps of MFMA work.  Rows past the
// end of the sequence are loaded from the last valid row and masked in the arithmetic.
// No atomics: each key row has one owner.
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

constexpr int kRows = 64;
constexpr int kCB = 1024 + 128;  // bytes per chunk column of a row tile (Q, dY)
constexpr int kVB = 1024;        // bytes per chunk column of the V tile (row reads only)
typedef __attribute__((address_space(3))) void lds_void;

struct DkvArgs {
  const uint16_t* q; const uint16_t* q_rope;
  const uint16_t* k; const uint16_t* k_rope;
  const uint16_t* v; const uint16_t* dy;
  const float* lse2; const float* drow;
  uint16_t* dk; uint16_t* dk_rope; uint16_t* dv;
  const int64_t* cu_q; const int64_t* cu_kv;
  const int32_t* tiles;  // (sequence, key tile), heaviest first
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
// unlike __syncthreads(), does not wait for this wave's outstanding global->LDS transfers
// (its release fence would).  Each wave first waits for the transfers it needs with
// wait_vmcnt; the step loop issues no ordinary LDS writes.
__device__ __forceinline__ void barrier_no_dma_wait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// global -> LDS transfers of one 16-byte (dma16) or 4-byte (dma4) element per lane.
// The immediate OFF is added to both addresses: lane l reads `src` + OFF and writes LDS
// byte M0 + OFF + l * size, with M0 = `lds` + MOFF (wave-uniform).  Issued through inline
// assembly so that the compiler does not add its own conservative waits; every wait on
// these transfers is an explicit wait_vmcnt.
__device__ __forceinline__ uint32_t lds_addr(const void* lds) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds);
}
template <int MOFF, int OFF>
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%3"
               ::"v"(src), "s"(lds), "i"(MOFF), "i"(OFF) : "memory", "m0", "scc");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
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

template <int DQK, int DV>
__global__ __launch_bounds__(256, 1) void kv_dense_kernel(DkvArgs a) {
  constexpr int KS = DQK / 32, VS = DV / 32, NQ = DQK / 16, NV = DV / 16;
  constexpr int QCH = DQK / 8, YCH = DV / 8;   // 16-byte chunks per row
  constexpr int QLD = QCH / 4, YLD = YCH / 4;  // transfer instructions per wave per tile
  constexpr int NLD = QLD + YLD + 2;           // + lse2, drow
  constexpr int QB = QCH * kCB, YB = YCH * kCB;
  __shared__ __attribute__((aligned(16))) char Q0[QB], Q1[QB], Q2[QB];
  __shared__ __attribute__((aligned(16))) char Y0[YB], Y1[YB], Y2[YB];
  __shared__ __attribute__((aligned(16))) float L0[kRows], L1[kRows], L2[kRows];
  __shared__ __attribute__((aligned(16))) float R0[kRows], R1[kRows], R2[kRows];
  __shared__ __attribute__((aligned(16))) char Vs[YCH * kVB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4, jj = l16 >> 2, qq = l16 & 3;

  const int b = a.tiles[2 * blockIdx.x];
  const int kt0 = a.tiles[2 * blockIdx.x + 1];
  const int kvh = blockIdx.y;
  const int64_t ks = a.cu_kv[b];
  const int S2 = (int)(a.cu_kv[b + 1] - ks);
  const int64_t k0 = ks + (int64_t)kt0 * kRows;
  const int nk = min(kRows, S2 - kt0 * kRows);
  const int64_t qs = a.cu_q[b];
  const int S1 = (int)(a.cu_q[b + 1] - qs);
  const int nqt = (S1 + kRows - 1) / kRows;
  const int qt0 = a.causal ? min(kt0, nqt) : 0;
  const int nq = nqt - qt0;
  const int nsteps = a.G * nq;
  const int qmain = a.d_main / 8;  // chunks of a Q row that come from `query` (the rest: queryRope)

  // ---- resident keys: K in registers (B of S = Q K^T), V in LDS (B of dP = dY V^T) ----
  bf16x8 Kf[KS];
  {
    const int key = 16 * w + l16;
    const bool valid = key < nk;
    const int64_t kr = (k0 + key) * a.n2 + kvh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int d = 32 * s + 8 * g;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (valid) x = ldg16(d < a.d_main ? a.k + kr * a.d_main + d : a.k_rope + kr * a.d_rope + (d - a.d_main));
      Kf[s] = __builtin_bit_cast(bf16x8, x);
    }
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      const int c = 4 * s + g;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (valid) x = ldg16(a.v + kr * a.d_v + 8 * c);
      sts16(&Vs[c * kVB + 16 * key], x);
    }
  }

  f32x4 dK[NQ], dV[NV];
#pragma unroll
  for (int n = 0; n < NQ; ++n) dK[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int n = 0; n < NV; ++n) dV[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Per-lane LDS byte offsets: row reads (rows 16rt + l16, chunk 4k + g) and column reads
  // (rows 32ks + 4g + jj (+16), chunk 2k + qq/2, byte half (qq&1)); the rest is immediate.
  const int rd_row = g * kCB + 16 * l16;
  const int rd_col = (qq >> 1) * kCB + 16 * (4 * g + jj) + 8 * (qq & 1);

  // Step st covers head hg = st / nq and query tile qt = qt0 + st % nq.
  // issue(): wave w moves chunks c = w + 4k of the 64 rows (lane = row) into one stage.
  // Chunk c of a row is 16 c bytes into the row and lands at c * kCB in the stage, so
  // with the per-lane row address + 16 w and the stage + w * kCB as bases, chunk k is the
  // immediate offset 64 k on the global side and 4 k kCB on the LDS side.
  const int kq = (qmain - w + 3) >> 2;  // chunks k < kq come from `query`, the rest from queryRope
  auto issue = [&](int st, const char* Qb, const char* Yb, const float* Lb, const float* Rb) {
    const int hg = st / nq;
    const int qt = qt0 + (st - hg * nq);
    const int h = kvh * a.G + hg;
    const int nvalid = min(kRows, S1 - qt * kRows);
    const int64_t r0 = qs + (int64_t)qt * kRows;
    const int64_t qr = (r0 + min(lane, nvalid - 1)) * a.n1 + h;
    const char* qrow = reinterpret_cast<const char*>(a.q + qr * a.d_main) + 16 * w;
    const char* rrow = reinterpret_cast<const char*>(a.q_rope + qr * a.d_rope) + 16 * (w - qmain);
    const char* yrow = reinterpret_cast<const char*>(a.dy + qr * a.d_v) + 16 * w;
    const uint32_t qb = lds_addr(Qb + w * kCB), yb = lds_addr(Yb + w * kCB);
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
    if (lane < 16) dma4(a.lse2 + lr, lds_addr(Lb + 16 * w));
    if (lane < 16) dma4(a.drow + lr, lds_addr(Rb + 16 * w));
  };

  auto step = [&](int st, const char* Qs, const char* Ys, const float* Ls, const float* Rs) {
    const int hg = st / nq;
    const int qt = qt0 + (st - hg * nq);
    const int nvalid = min(kRows, S1 - qt * kRows);

    // S = Q K^T, dP = dY V^T: items i = (k-step gi, row tile rt), A fragments PD1 ahead
    constexpr int NI1 = 4 * (KS + VS), PD1 = 6;
    f32x4 S[4], D[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) { S[rt] = f32x4{0.f, 0.f, 0.f, 0.f}; D[rt] = S[rt]; }
    auto a1 = [&](int i) -> bf16x8 {
      const int gi = i >> 2, rt = i & 3;
      return gi < KS ? *at_bytes<bf16x8>(Qs, rd_row + 4 * gi * kCB + 256 * rt)
                     : *at_bytes<bf16x8>(Ys, rd_row + 4 * (gi - KS) * kCB + 256 * rt);
    };
    bf16x8 ring1[PD1];
#pragma unroll
    for (int i = 0; i < PD1; ++i) ring1[i] = a1(i);
    bf16x8 vb[VS];
#pragma unroll
    for (int s = 0; s < VS; ++s) vb[s] = *at_bytes<bf16x8>(Vs, (4 * s + g) * kVB + 16 * (16 * w + l16));
#pragma unroll
    for (int i = 0; i < NI1; ++i) {
      const int gi = i >> 2, rt = i & 3;
      const bf16x8 x = ring1[i % PD1];
      if (i + PD1 < NI1) ring1[i % PD1] = a1(i + PD1);
      if (gi < KS) S[rt] = mfma_16x16x32(x, Kf[gi], S[rt]);
      else D[rt] = mfma_16x16x32(x, vb[gi - KS], D[rt]);
    }
    // P and dS in place (mask: causal, ragged tail of the query tile)
    const int key = kt0 * kRows + 16 * w + l16;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const f32x4 lse = *reinterpret_cast<const f32x4*>(&Ls[16 * rt + 4 * g]);
      const f32x4 dr = *reinterpret_cast<const f32x4*>(&Rs[16 * rt + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        float p = __builtin_amdgcn_exp2f(S[rt][i] * a.scale_log2e - lse[i]);
        const bool masked = r >= nvalid || (a.causal && key > qt * kRows + r);
        p = masked ? 0.f : p;
        D[rt][i] = p * (D[rt][i] - dr[i]);
        S[rt][i] = p;
      }
    }
    // dV += P^T dY, dK += dS^T Q: items i = (half ks, output tile j), column fragments PD2 ahead
    const bf16x8 pa[2] = {pack8(S[0], S[1]), pack8(S[2], S[3])};
    const bf16x8 da[2] = {pack8(D[0], D[1]), pack8(D[2], D[3])};
    constexpr int NJ = NV + NQ, NI2 = 2 * NJ, PD2 = 6;
    auto b2 = [&](int i) -> bf16x8 {
      const int ks2 = i / NJ, j = i - (i / NJ) * NJ;
      const char* base = j < NV ? Ys : Qs;
      const int jt = j < NV ? j : j - NV;
      const int o = rd_col + 2 * jt * kCB + 16 * 32 * ks2;
      return join8(lds_read_tr16(reinterpret_cast<const uint16_t*>(base + o)),
                   lds_read_tr16(reinterpret_cast<const uint16_t*>(base + o + 16 * 16)));
    };
    bf16x8 ring2[PD2];
#pragma unroll
    for (int i = 0; i < PD2; ++i) ring2[i] = b2(i);
#pragma unroll
    for (int i = 0; i < NI2; ++i) {
      const int ks2 = i / NJ, j = i - (i / NJ) * NJ;
      const bf16x8 bv = ring2[i % PD2];
      if (i + PD2 < NI2) ring2[i % PD2] = b2(i + PD2);
      if (j < NV) dV[j] = mfma_16x16x32(pa[ks2], bv, dV[j]);
      else dK[j - NV] = mfma_16x16x32(da[ks2], bv, dK[j - NV]);
    }
  };

  __syncthreads();  // V tile stored; nothing is in flight yet
  if (nsteps > 0) issue(0, Q0, Y0, L0, R0);
  if (nsteps > 1) issue(1, Q1, Y1, L1, R1);
  for (int st = 0; st < nsteps; ++st) {
    // stage st has landed once at most one later stage is still in flight
    if (st + 1 < nsteps) wait_vmcnt<NLD>();
    else wait_vmcnt<0>();
    barrier_no_dma_wait();  // every wave's share of stage st is in LDS; stage st-1 is free
    switch (st % 3) {
      case 0:
        if (st + 2 < nsteps) issue(st + 2, Q2, Y2, L2, R2);
        step(st, Q0, Y0, L0, R0);
        break;
      case 1:
        if (st + 2 < nsteps) issue(st + 2, Q0, Y0, L0, R0);
        step(st, Q1, Y1, L1, R1);
        break;
      default:
        if (st + 2 < nsteps) issue(st + 2, Q1, Y1, L1, R1);
        step(st, Q2, Y2, L2, R2);
        break;
    }
  }

  // ---- epilogue: bf16 through LDS (chunk-major), 16-byte stores ----------------------
  __syncthreads();
  uint16_t* Ko = reinterpret_cast<uint16_t*>(Q0);
  uint16_t* Vo = reinterpret_cast<uint16_t*>(Y0);
#pragma unroll
  for (int nt = 0; nt < NQ; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * g + i, col = 16 * nt + l16;
      Ko[((col >> 3) * kCB + 16 * r) / 2 + (col & 7)] = f2bf(dK[nt][i] * a.scale);
    }
#pragma unroll
  for (int nt = 0; nt < NV; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * g + i, col = 16 * nt + l16;
      Vo[((col >> 3) * kCB + 16 * r) / 2 + (col & 7)] = f2bf(dV[nt][i]);
    }
  __syncthreads();
  for (int idx = tid; idx < kRows * QCH; idx += 256) {
    const int r = idx / QCH, c = idx - r * QCH, d = 8 * c;
    if (r < nk) {
      const int64_t kr = (k0 + r) * a.n2 + kvh;
      uint16_t* dst = d < a.d_main ? a.dk + kr * a.d_main + d : a.dk_rope + kr * a.d_rope + (d - a.d_main);
      sts16(dst, *at_bytes<uint4>(Q0, c * kCB + 16 * r));
    }
  }
  for (int idx = tid; idx < kRows * YCH; idx += 256) {
    const int r = idx / YCH, c = idx - r * YCH;
    if (r < nk) sts16(a.dv + ((k0 + r) * a.n2 + kvh) * a.d_v + 8 * c, *at_bytes<uint4>(Y0, c * kCB + 16 * r));
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
  k.cu_q = a.cu_q; k.cu_kv = a.cu_kv; k.tiles = a.kv_tiles;
  k.n1 = a.n1; k.n2 = a.n2; k.G = a.G;
  k.d_main = a.d_main; k.d_rope = a.d_rope; k.d_v = a.d_v;
  k.causal = a.causal; k.scale = a.scale; k.scale_log2e = a.scale_log2e;
  const dim3 grid(a.n_kv_tiles, a.n2);
  const int dqk = a.d_main + a.d_rope;
  if (dqk == 192 && a.d_v == 128) hipLaunchKernelGGL((kv_dense_kernel<192, 128>), grid, dim3(256), 0, s, k);
  else if (dqk == 128 && a.d_v == 128) hipLaunchKernelGGL((kv_dense_kernel<128, 128>), grid, dim3(256), 0, s, k);
  else if (dqk == 64 && a.d_v == 64) hipLaunchKernelGGL((kv_dense_kernel<64, 64>), grid, dim3(256), 0, s, k);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ab
