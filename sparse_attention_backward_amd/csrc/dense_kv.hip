// Dense KV-major backward: dK and dV accumulated in registers, plus the dS tiles that
// the dQ product consumes (bf16 MFMA, fp32 accumulation).
//
// Page "aclnnFlashAttentionUnpaddingScoreGradV3", Formula section: dV = P^T dY,
// dK = dS^T Q / sqrt(d), dkRope = dS^T qRope / sqrt(d), with Q = [query, queryRope].
//
// One workgroup (8 waves) owns a 128-key tile of one sequence and KV head, and a range of
// its query tiles.  Query rows stream past in steps of 64 rows: the query tiles of the
// range from the last one down, each for the G query heads of the KV head in turn.
// Walking every key tile's list from the same end keeps the workgroups of one
// (sequence, KV head) on the same query tile at the same time, so their row loads share
// the L2.
//
// Waves w and w + 4 own keys 32(w%4) .. +31 of the tile and split each 32-row half step
// between them (two waves per SIMD, one of each kind, so that one wave's LDS waits and
// exponentials overlap the other's matrix work):
//   S wave (w < 4), K resident:   S = Q K^T; P = exp2(S*scale*log2e - lse2) with the masks
//                                 (edges of the causal / window mask, ragged query tail);
//                                 P -> LDS;
//                                 dV += P^T dY
//   dP wave (w >= 4), V resident: dP = dY V^T; dS = P (dP - drow) with P from LDS;
//                                 dS^T -> workspace (bf16, one 64 x 64 block per (query
//                                 tile, 64-key tile, head)); dK += dS^T Q
// A operands of S / dP: Q / dY rows from LDS (16-byte reads); of dV / dK: the P / dS C
// tiles repacked in registers; B operands of dV / dK: dY / Q columns (ds_read_b64_tr_b16).
// Each kind does 2*(D_qk + D_v) flop per (row, key) pair.  The dP waves work one step
// behind the S waves: step s's P, written before barrier s + 1, is read after it.
// Masks (causal, windows): a 32-key block against a 32-row block is skipped when none of its
// pairs is visible, masked element by element when it crosses an edge of the mask, and
// complete otherwise.
//
// Key tiles with many query tiles are split into ranges (so that no workgroup runs far
// longer than the average): each range leaves its fp32 dK / dV in a partial slot, in
// register order, and the first workgroups of the dQ launch add the ranges of a tile in
// range order.
// Every output row has one writer: no atomics, deterministic.
//
// Staging: a step's Q (query and queryRope parts), dY, lse2 and ndrow go from global memory
// straight into one of three LDS stages (global_load_lds), issued one step ahead; the
// stage of step s is read by the S waves in iteration s and by the dP waves in iteration
// s + 1.  Each part is a RowTile: every transfer instruction reads whole rows (full cache
// lines) into one 1 KB block, and the chunk swizzle keeps the row / column reads conflict
// free.
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

constexpr int kRows = 64;                // query rows per step, rows / keys of a dS block
constexpr int kKeys = kDenseKeyTile;     // keys per workgroup
typedef __attribute__((address_space(3))) void lds_void;

struct DkvArgs {
  const uint16_t* q; const uint16_t* q_rope;
  const uint16_t* k; const uint16_t* k_rope;
  const uint16_t* v; const uint16_t* dy;
  const float* lse2; const float* ndrow;
  uint16_t* dk; uint16_t* dk_rope; uint16_t* dv;
  uint16_t* ds;               // [block][head][64 keys][64 rows] bf16 (dS transposed)
  const int64_t* cu_q; const int64_t* cu_kv;
  const int32_t* qt_base;     // [B + 1] query tiles before each sequence
  const int64_t* qt_blk;      // first stored dS block of each query tile
  const int32_t* qt_kr;       // [query tiles][2] its 64-key tiles [lo, hi)
  const int32_t* tiles;       // [n][6] (sequence, 128-key tile, KV head, first / end query tile,
                              // partial slot or -1); sequence < 0: idle slot
  const int32_t* split;       // [n][5] (sequence, 128-key tile, KV head, first slot, parts)
  float* part;                // fp32 partials, kDenseKvPartBytes per slot
  int n1, n2, G;
  int lo_rel, hi_rel, align;  // mask on j - i (dense_band); unbounded without a mask
  float scale, scale_log2e;
};

// Workgroup barrier that keeps the compiler from moving memory accesses across it; each
// wave first waits for its own transfers and LDS accesses.
__device__ __forceinline__ void barrier_all_done() {
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16 bytes per lane from global memory into LDS at (M0 = lds + MOFF) + 16 * lane
template <int MOFF>
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               ::"v"(src), "s"(lds), "i"(MOFF) : "memory", "m0", "scc");
}

// The same from base + voff (a wave-uniform 64-bit base and a per-lane 32-bit offset)
template <int MOFF>
__device__ __forceinline__ void dma16s(uint32_t voff, const void* base, uint32_t lds) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               ::"v"(voff), "s"(base), "s"(lds), "i"(MOFF) : "memory", "m0", "scc");
}

// 4 bytes per lane from global memory into LDS at M0 = lds, + 4 * lane
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               ::"v"(src), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* lds) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds);
}

template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

// Per-lane addressing of one staged part (a RowTile of W chunks per row).
//   transfers: S wave w (of 4) fills 1 KB blocks i = w + 4k (k < W/4) of the part; lane l
//              fills row i RPI + l / W, slot l % W, i.e. reads chunk (l % W) ^ swz(row) --
//              the same chunk for every k, because 4 RPI rows is a multiple of 16.
//   row reads (A operands): rows 16rt + l16, chunk 4s + g (+32 rows for the second half).
//   column reads (transposed, B operands): rows 4g + jj (+16), chunk 2j + qq/2, half qq&1
//              (+32 rows for the second half).
template <int W>
struct PartLanes {
  using T = RowTile<W>;
  static_assert(W % 4 == 0, "whole blocks per wave");
  int row0;          // transfer row for k = 0
  uint32_t gchunk;   // byte offset of the chunk this lane reads within its row
  __device__ __forceinline__ void init(int w, int lane) {
    row0 = w * T::RPI + lane / W;
    gchunk = 16u * (uint32_t)((lane % W) ^ T::swz(row0));
  }
  __host__ __device__ static constexpr int rowA(int lane, int s) { return T::rowA(lane, s); }
  __host__ __device__ static constexpr int colB(int lane, int j) { return T::colB(lane, j); }
};

// Accumulators of one kind (dK: S = 0 unused, or dV) of this pair's 32 keys to bf16 rows
// in LDS (rows 32p .. +31 of a [128][D] tile at lds), scaled by sc.
template <int D>
__device__ __forceinline__ void acc_to_lds(uint16_t* tile, const f32x4 (&acc)[2][D / 16], int p, int lane, float sc) {
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) tile[(32 * p + 16 * t + 4 * g + i) * D + 16 * n + l16] = f2bf(acc[t][n][i] * sc);
}

// bf16 rows r < nk of the [128][DQK] dK and [128][DV] dV tiles in LDS to global memory.
template <int DM, int DR, int DV>
__device__ __forceinline__ void tiles_to_global(const DkvArgs& a, const uint16_t* Ko, const uint16_t* Vo, int tid,
                                                int nthreads, int64_t k0, int nk, int kvh) {
  constexpr int DQK = DM + DR, QCH = DQK / 8, YCH = DV / 8;
  for (int idx = tid; idx < kKeys * QCH; idx += nthreads) {
    const int r = idx / QCH, c = idx - r * QCH, d = 8 * c;
    if (r < nk) {
      const int64_t kr = (k0 + r) * a.n2 + kvh;
      uint16_t* dst = d < DM ? a.dk + kr * DM + d : a.dk_rope + kr * DR + (d - DM);
      sts16(dst, *reinterpret_cast<const uint4*>(Ko + r * DQK + d));
    }
  }
  for (int idx = tid; idx < kKeys * YCH; idx += nthreads) {
    const int r = idx / YCH, c = idx - r * YCH;
    if (r < nk) sts16(a.dv + ((k0 + r) * a.n2 + kvh) * DV + 8 * c, *reinterpret_cast<const uint4*>(Vo + r * DV + 8 * c));
  }
}

template <int DM, int DR, int DV, bool DS>
__global__ __launch_bounds__(512, 1) void dense_kv_kernel(DkvArgs a) {
  constexpr int DQK = DM + DR;
  constexpr int KS = DQK / 32, VS = DV / 32, NQ = DQK / 16, NV = DV / 16;
  constexpr int KSM = DM / 32, NQM = DM / 16;  // k-steps / column tiles of the query part
  constexpr int WM = DM / 8, WR = DR > 0 ? DR / 8 : 8, WY = DV / 8;
  using TM = RowTile<WM>;
  using TR = RowTile<WR>;
  using TY = RowTile<WY>;
  // stage: QM, QR, Y, lse2 (64 floats), ndrow (64 floats); three stages, then the P
  // exchange: [step parity][pair][half] 2 KB (two 1 KB arrays of 16 bytes per lane)
  constexpr int OQM = 0, OQR = TM::BYTES, OY = OQR + (DR > 0 ? TR::BYTES : 0);
  constexpr int OL = OY + TY::BYTES, SB = OL + 512;
  constexpr int OX = 3 * SB, XBYTES = 2 * 4 * 2 * 2048;
  constexpr int EPI = kKeys * (DQK + DV) * 2;  // epilogue: bf16 output tiles
  constexpr int SMEM = OX + XBYTES > EPI ? OX + XBYTES : EPI;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  static_assert(SB % 256 == 0 && OQR % 256 == 0 && OY % 256 == 0, "part bases keep bits 0-7 clear");
  static_assert(2 * (NQ + NV) * 16 * 256 <= kDenseKvPartBytes, "partial slot size");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p = w & 3;            // key pair: keys 32p .. +31 of the tile
  const bool swave = w < 4;
  const int l16 = lane & 15, g = lane >> 4;

  const int32_t* tl = a.tiles + 6 * blockIdx.x;
  const int b = tl[0];
  if (b < 0) return;  // idle slot of the schedule
  const int kt0 = tl[1], kvh = tl[2], qa = tl[3], qb = tl[4], slot = tl[5];
  const int64_t ks = a.cu_kv[b];
  const int S2 = (int)(a.cu_kv[b + 1] - ks);
  const int64_t k0 = ks + (int64_t)kt0 * kKeys;
  const int nk = min(kKeys, S2 - kt0 * kKeys);
  const int nkt64 = (S2 + kRows - 1) / kRows;
  const int64_t qs = a.cu_q[b];
  const int S1 = (int)(a.cu_q[b + 1] - qs);
  const int nsteps = a.G * (qb - qa);
  int mlo, mhi;  // key j visible to query i iff mlo <= j - i <= mhi (positions in the sequence)
  dense_band(a.lo_rel, a.hi_rel, a.align, S1, S2, mlo, mhi);
  const int kb = 4 * kt0 + p;           // this pair's 32-key block
  const int kt64 = 2 * kt0 + (p >> 1);  // its 64-key tile (dS block column)
  const bool idle = 32 * p >= nk;       // every key of this pair lies past the sequence

  // step st -> (query tile qt, head hg): the range's query tiles from the last one down,
  // the G heads of a query tile back to back
  auto step_tile = [&](int st, int& hg, int& qt) {
    const int i = st / a.G;
    hg = st - i * a.G;
    qt = qb - 1 - i;
  };

  const uint32_t smem_lds = lds_addr(smem);
  const uint32_t rs_m = (uint32_t)a.n1 * DM * 2, rs_r = (uint32_t)a.n1 * DR * 2, rs_y = (uint32_t)a.n1 * DV * 2;
  PartLanes<WM> pm;
  PartLanes<WR> pr;
  PartLanes<WY> py;
  pm.init(w, lane);
  if constexpr (DR > 0) pr.init(w, lane);
  py.init(w, lane);
  const uint32_t vo_m = (uint32_t)pm.row0 * rs_m + pm.gchunk, vo_y = (uint32_t)py.row0 * rs_y + py.gchunk;
  const uint32_t vo_r = DR > 0 ? (uint32_t)pr.row0 * rs_r + pr.gchunk : 0u;

  // Transfers of step st into the stage at LDS address stage, issued by the S waves only
  // (so that the dP waves never wait for vector-memory counts and their dS stores stay in
  // flight across barriers): this wave's blocks of each part (rows past the end of the
  // sequence repeat its last row), and the lse2 (wave 0) or ndrow (wave 1) values of the 64
  // rows.
  // With every row of the step in the sequence, transfer k reads rows 4 RPI k further on: a
  // wave-uniform base and the lane's fixed offset voff (no per-transfer vector arithmetic).
  auto issue_part = [&](auto wtag, const auto& pl, uint32_t voff, const char* gtile, uint32_t rs, uint32_t lds_part,
                        int nvalid) {
    constexpr int W = decltype(wtag)::value;
    constexpr int RPI = RowTile<W>::RPI;
    if (nvalid == kRows) {
      static_for<W / 4>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        dma16s<4096 * k>(voff, gtile + (size_t)(4 * RPI * k) * rs, lds_part + w * 1024);
      });
    } else {
      static_for<W / 4>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const int r = min(pl.row0 + 4 * RPI * k, nvalid - 1);
        dma16<4096 * k>(gtile + __umul24((uint32_t)r, rs) + pl.gchunk, lds_part + w * 1024);
      });
    }
  };
  auto issue_stage = [&](int st, uint32_t stage) {
    int hg, qt;
    step_tile(st, hg, qt);
    const int nvalid = min(kRows, S1 - qt * kRows);
    const int64_t rh0 = (qs + (int64_t)qt * kRows) * a.n1 + kvh * a.G + hg;  // (first row) * n1 + h
    issue_part(std::integral_constant<int, WM>{}, pm, vo_m, reinterpret_cast<const char*>(a.q + rh0 * DM), rs_m,
               stage + OQM, nvalid);
    if constexpr (DR > 0)
      issue_part(std::integral_constant<int, WR>{}, pr, vo_r, reinterpret_cast<const char*>(a.q_rope + rh0 * DR), rs_r,
                 stage + OQR, nvalid);
    issue_part(std::integral_constant<int, WY>{}, py, vo_y, reinterpret_cast<const char*>(a.dy + rh0 * DV), rs_y,
               stage + OY, nvalid);
    if (w < 2) {
      const int64_t lrow = rh0 + (int64_t)min(lane, nvalid - 1) * a.n1;
      dma4(w == 0 ? a.lse2 + lrow : a.ndrow + lrow, stage + OL + 256 * w);
    }
  };
  auto stage_of = [&](int st) { return smem_lds + (uint32_t)(st % 3) * SB; };
  auto xslot = [&](int st, int hi) { return smem_lds + OX + (uint32_t)((((st & 1) * 4 + p) * 2 + hi) * 2048); };
  // the pair's 32-key block against the 32-row block of half hh of step st: skipped when no
  // (key, row) pair of it is visible (j - i spans 32 (kb - rb) - 31 .. + 31)
  auto half_active = [&](int st, int hh, int& hg, int& qt, int& rb) {
    step_tile(st, hg, qt);
    rb = 2 * qt + hh;
    const int d0 = 32 * (kb - rb);
    return !idle && d0 + 31 >= mlo && d0 - 31 <= mhi;
  };

  if (nsteps > 0 && swave) issue_stage(0, smem_lds);

  if (swave) {
    // ---------------- S waves: S, P, dV -------------------------------------------------
    bf16x8 Kf[2][KS];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = 32 * p + 16 * t + l16;
      const bool valid = key < nk;
      const int64_t kr = (k0 + key) * a.n2 + kvh;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int d = 32 * s + 8 * g;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (valid) x = ldg16(d < DM ? a.k + kr * DM + d : a.k_rope + kr * DR + (d - DM));
        Kf[t][s] = __builtin_bit_cast(bf16x8, x);
      }
    }
    f32x4 dV[2][NV];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int n = 0; n < NV; ++n) dV[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto s_half = [&](int st, uint32_t stage, auto hic) {
      constexpr int hi = decltype(hic)::value;
      int hg, qt, rb;
      if (!half_active(st, hi, hg, qt, rb)) return;
      const int d0 = 32 * (kb - rb);
      const bool edge = d0 - 31 < mlo || d0 + 31 > mhi;  // the block crosses an edge of the mask
      const int nvalid = min(kRows, S1 - qt * kRows);
      const uint32_t vm = stage + OQM + PartLanes<WM>::rowA(lane, 0), vr = stage + OQR + PartLanes<WR>::rowA(lane, 0);
      const uint32_t vy = stage + OY + PartLanes<WY>::colB(lane, 0);
      const uint32_t statb = opaque(stage + OL + 4 * (32 * hi + 4 * g));
      f32x4 lse[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) lse[rt] = lds_f32x4_at(statb + 64 * rt);
      if (nvalid < kRows) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) lse[rt][i] = 32 * hi + 16 * rt + 4 * g + i < nvalid ? lse[rt][i] : INFINITY;
      }
      // S = Q K^T: k-steps s < KSM over the query part, the rest over the rope part; the A
      // fragments of a k-step (both row tiles) serve both key tiles and are read PA ahead
      constexpr int PA = 2;
      auto afrag = [&](int s, int rt) -> bf16x8 {
        if (s < KSM) return lds_b128_at((vm ^ (64u * s)) + (32 * hi + 16 * rt) * TM::RB);
        return lds_b128_at((vr ^ (64u * (s - KSM))) + (32 * hi + 16 * rt) * TR::RB);
      };
      bf16x8 aring[PA][2];
#pragma unroll
      for (int i = 0; i < PA; ++i) { aring[i][0] = afrag(i, 0); aring[i][1] = afrag(i, 1); }
      f32x4 S[2][2];  // [key tile][row tile]
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 a0 = aring[s % PA][0], a1 = aring[s % PA][1];
        if (s + PA < KS) { aring[s % PA][0] = afrag(s + PA, 0); aring[s % PA][1] = afrag(s + PA, 1); }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          S[t][0] = mfma_16x16x32(a0, Kf[t][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : S[t][0]);
          S[t][1] = mfma_16x16x32(a1, Kf[t][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : S[t][1]);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * PA, 0);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        if (s + PA < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) S[t][rt][i] = __builtin_amdgcn_exp2f(S[t][rt][i] * a.scale_log2e - lse[rt][i]);
      if (edge) {
        // key 32kb + 16t + l16 against row 32rb + 16rt + 4g + i: j - i = d0 + 16(t - rt) + l16 - 4g - i
        const int dl = d0 + l16 - 4 * g;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int d = dl + 16 * (t - rt) - i;
              S[t][rt][i] = (d < mlo || d > mhi) ? 0.f : S[t][rt][i];
            }
      }
      // P as bf16 for this wave's dV product and as f16 (more mantissa, and the dP wave's
      // mixed-precision multiply takes f16 halves directly) for the exchange
      bf16x8 pa[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) pa[t] = pack8(S[t][0], S[t][1]);
      const uint32_t xs = xslot(st, hi) + 16 * lane;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint32_t h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          h[q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(S[t][q >> 1][2 * (q & 1)], S[t][q >> 1][2 * (q & 1) + 1]));
        lds_st16_at(xs + 1024 * t, make_uint4(h[0], h[1], h[2], h[3]));
      }
      // dV += P^T dY: column fragments of dY (two transposed reads each), PD items ahead
      auto colfrag = [&](int j) -> bf16x8 {
        const uint32_t o = vy ^ (32u * j);
        return join8(lds_tr16_at(o + 32 * hi * TY::RB), lds_tr16_at(o + (32 * hi + 16) * TY::RB));
      };
      constexpr int PD = 4;
      bf16x8 ring[PD];
#pragma unroll
      for (int i = 0; i < PD; ++i) ring[i] = colfrag(i);
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const bf16x8 bj = ring[j % PD];
        if (j + PD < NV) ring[j % PD] = colfrag(j + PD);
        dV[0][j] = mfma_16x16x32(pa[0], bj, dV[0][j]);
        dV[1][j] = mfma_16x16x32(pa[1], bj, dV[1][j]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * PD, 1);
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
        if (j + PD < NV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
    };

    for (int st = 0; st <= nsteps; ++st) {
      barrier_all_done();
      if (st + 1 < nsteps) issue_stage(st + 1, stage_of(st + 1));
      if (st < nsteps) {
        const uint32_t stage = stage_of(st);
        s_half(st, stage, std::integral_constant<int, 0>{});
        s_half(st, stage, std::integral_constant<int, 1>{});
      }
    }

    // ---- epilogue: dV ----
    if (slot < 0) {
      __syncthreads();  // LDS free
      acc_to_lds<DV>(reinterpret_cast<uint16_t*>(smem) + kKeys * DQK, dV, p, lane, 1.f);
      __syncthreads();
    } else {
      f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<char*>(a.part) + (size_t)slot * kDenseKvPartBytes) +
                   p * (2 * (NQ + NV)) * 64 + lane;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int n = 0; n < NV; ++n) dst[(t * (NQ + NV) + NQ + n) * 64] = dV[t][n];
    }
  } else {
    // ---------------- dP waves: dP, dS, dK (one step behind) ----------------------------
    // The dP waves carry the longer part of a step (their dS arithmetic and stores); the S
    // waves wait at the barrier meanwhile, so the dP waves get issue priority on the SIMD.
    __builtin_amdgcn_s_setprio(3);
    bf16x8 Vf[2][VS];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = 32 * p + 16 * t + l16;
      const bool valid = key < nk;
      const int64_t kr = (k0 + key) * a.n2 + kvh;
#pragma unroll
      for (int s = 0; s < VS; ++s) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (valid) x = ldg16(a.v + kr * DV + 32 * s + 8 * g);
        Vf[t][s] = __builtin_bit_cast(bf16x8, x);
      }
    }
    f32x4 dK[2][NQ];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int n = 0; n < NQ; ++n) dK[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // dS^T of one step: rows (keys) 32(p&1) + 16t + l16 of the 64-key tile, all 64 columns
    // (query rows).  After half step hi a lane holds, per key tile, the 4-column pieces
    // 8hi + g (columns 32hi + 4g ..) and 8hi + 4 + g (+16).  One lane swap between rows g and
    // g ^ 1 of the wave (v_permlane16_swap: an even row keeps its first operand and receives
    // the odd row's first; an odd row receives the even row's second and keeps its own)
    // leaves every lane two adjacent pieces, 16 bytes: pieces 8hi + {g, g + 1} for even g,
    // 8hi + {g + 3, g + 4} for odd g, so the four lanes of a key row write 64 contiguous bytes
    // per half.  Zeros for keys past the end of the sequence.
    auto pair_pieces = [&](const bf16x8& d) -> u32x4 {
      const u32x4 v = __builtin_bit_cast(u32x4, d);
      const auto s0 = __builtin_amdgcn_permlane16_swap(v[0], v[2], false, false);
      const auto s1 = __builtin_amdgcn_permlane16_swap(v[1], v[3], false, false);
      return u32x4{s0[0], s1[0], s0[1], s1[1]};
    };
    const int piece_col = (g & 1) ? 4 * g + 12 : 4 * g;
    auto store_ds = [&](uint16_t* row, const u32x4 (&c0)[2], const u32x4 (&c1)[2]) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 x0 = c0[t], x1 = c1[t];
        if (nk < kKeys && 32 * p + 16 * t + l16 >= nk) x0 = x1 = u32x4{0u, 0u, 0u, 0u};
        // streaming stores: the dS blocks are read back only by the next kernel, so they
        // should not push the query rows that other key tiles still read out of the L2
        __builtin_nontemporal_store(x0, reinterpret_cast<u32x4*>(row + 16 * t * kRows + piece_col));
        __builtin_nontemporal_store(x1, reinterpret_cast<u32x4*>(row + 16 * t * kRows + 32 + piece_col));
      }
    };

    // The dS^T row of this lane's key in the block of step st, or nullptr when no block
    // exists (no key of the 64-key tile is visible to a row of the query tile).
    auto ds_row = [&](int st) -> uint16_t* {
      int hg, qt;
      step_tile(st, hg, qt);
      const int gq = a.qt_base[b] + qt;
      const int klo = a.qt_kr[2 * gq], khi = a.qt_kr[2 * gq + 1];
      if (!(kt64 < nkt64 && kt64 >= klo && kt64 < khi)) return nullptr;
      const int64_t blk = a.qt_blk[gq] + (kt64 - klo);
      return a.ds + (blk * a.n1 + kvh * a.G + hg) * (int64_t)(kRows * kRows) + (32 * (p & 1) + l16) * kRows;
    };

    // A half step leaves its dS in da: zero where the pair's block is skipped.
    auto dp_half = [&](int st, uint32_t stage, auto hic, bf16x8 (&da)[2]) {
      constexpr int hi = decltype(hic)::value;
      int hg, qt, rb;
      const bool active = half_active(st, hi, hg, qt, rb);
      da[0] = da[1] = bf16x8{};
      if (!active) return;
      const uint32_t vm = stage + OQM + PartLanes<WM>::colB(lane, 0), vr = stage + OQR + PartLanes<WR>::colB(lane, 0);
      const uint32_t vy = stage + OY + PartLanes<WY>::rowA(lane, 0);
      const uint32_t statb = opaque(stage + OL + 256 + 4 * (32 * hi + 4 * g));
      const uint32_t xs = xslot(st, hi) + 16 * lane;
      const f16x8 p0 = lds_f16x8_at(xs), p1 = lds_f16x8_at(xs + 1024);
      f32x4 ndr[2];  // the dP accumulators start at ndrow = -drow, so they end at dP - drow
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) ndr[rt] = lds_f32x4_at(statb + 64 * rt);
      // dP = dY V^T over VS k-steps of dY rows
      constexpr int PA = 3;
      auto afrag = [&](int s, int rt) -> bf16x8 { return lds_b128_at((vy ^ (64u * s)) + (32 * hi + 16 * rt) * TY::RB); };
      bf16x8 aring[PA][2];
#pragma unroll
      for (int i = 0; i < PA; ++i) { aring[i][0] = afrag(i, 0); aring[i][1] = afrag(i, 1); }
      f32x4 D[2][2];  // [key tile][row tile]
#pragma unroll
      for (int s = 0; s < VS; ++s) {
        const bf16x8 a0 = aring[s % PA][0], a1 = aring[s % PA][1];
        if (s + PA < VS) { aring[s % PA][0] = afrag(s + PA, 0); aring[s % PA][1] = afrag(s + PA, 1); }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          D[t][0] = mfma_16x16x32(a0, Vf[t][s], s == 0 ? ndr[0] : D[t][0]);
          D[t][1] = mfma_16x16x32(a1, Vf[t][s], s == 0 ? ndr[1] : D[t][1]);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * PA + 2, 0);
#pragma unroll
      for (int s = 0; s < VS; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        if (s + PA < VS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      // dS = P (dP - drow); P is the S wave's f16 tile, in the same lane layout
      const f16x8 pp[2] = {p0, p1};
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 ds[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) ds[rt][i] = __builtin_fmaf((float)pp[t][4 * rt + i], D[t][rt][i], 0.f);
        da[t] = pack8(ds[0], ds[1]);
      }
      // dK += dS^T Q: column fragments of the query part, then of the rope part
      auto colfrag = [&](int j) -> bf16x8 {
        if (j < NQM) {
          const uint32_t o = vm ^ (32u * j);
          return join8(lds_tr16_at(o + 32 * hi * TM::RB), lds_tr16_at(o + (32 * hi + 16) * TM::RB));
        }
        const uint32_t o = vr ^ (32u * (j - NQM));
        return join8(lds_tr16_at(o + 32 * hi * TR::RB), lds_tr16_at(o + (32 * hi + 16) * TR::RB));
      };
      constexpr int PD = 3;
      bf16x8 ring[PD];
#pragma unroll
      for (int i = 0; i < PD; ++i) ring[i] = colfrag(i);
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const bf16x8 bj = ring[j % PD];
        if (j + PD < NQ) ring[j % PD] = colfrag(j + PD);
        dK[0][j] = mfma_16x16x32(da[0], bj, dK[0][j]);
        dK[1][j] = mfma_16x16x32(da[1], bj, dK[1][j]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * PD, 1);
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
        if (j + PD < NQ) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
    };

    // Iteration st handles step st - 1 and stores its dS^T rows at the end.  The barrier
    // waits only for this wave's LDS accesses: its stores stay in flight.
    for (int st = 0; st <= nsteps; ++st) {
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (st > 0) {
        const uint32_t stage = stage_of(st - 1);
        bf16x8 da[2];
        u32x4 c0[2], c1[2];
        dp_half(st - 1, stage, std::integral_constant<int, 0>{}, da);
        if constexpr (DS) {
#pragma unroll
          for (int t = 0; t < 2; ++t) c0[t] = pair_pieces(da[t]);
        }
        dp_half(st - 1, stage, std::integral_constant<int, 1>{}, da);
        if constexpr (DS) {
          uint16_t* row = ds_row(st - 1);
          if (row != nullptr) {
#pragma unroll
            for (int t = 0; t < 2; ++t) c1[t] = pair_pieces(da[t]);
            store_ds(row, c0, c1);
          }
        }
      }
    }

    // ---- epilogue: dK (scaled) ----
    if (slot < 0) {
      __syncthreads();  // LDS free
      acc_to_lds<DQK>(reinterpret_cast<uint16_t*>(smem), dK, p, lane, a.scale);
      __syncthreads();
    } else {
      f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<char*>(a.part) + (size_t)slot * kDenseKvPartBytes) +
                   p * (2 * (NQ + NV)) * 64 + lane;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int n = 0; n < NQ; ++n) dst[(t * (NQ + NV) + n) * 64] = dK[t][n];
    }
  }
  if (slot < 0)
    tiles_to_global<DM, DR, DV>(a, reinterpret_cast<const uint16_t*>(smem),
                                reinterpret_cast<const uint16_t*>(smem) + kKeys * DQK, tid, 512, k0, nk, kvh);
}

template <int DM, int DR, int DV>
hipError_t launch_kv(const DkvArgs& k, int n_tiles, bool ds, hipStream_t s) {
  if (ds) hipLaunchKernelGGL((dense_kv_kernel<DM, DR, DV, true>), dim3(n_tiles), dim3(512), 0, s, k);
  else hipLaunchKernelGGL((dense_kv_kernel<DM, DR, DV, false>), dim3(n_tiles), dim3(512), 0, s, k);
  return hipGetLastError();
}

}  // namespace

bool dense_bf16_supported(int d_main, int d_rope, int d_v) {
  return (d_main == 128 && d_rope == 64 && d_v == 128) || (d_main == 128 && d_rope == 0 && d_v == 128) ||
         (d_main == 64 && d_rope == 0 && d_v == 64);
}

hipError_t launch_dense_kv_bf16(const DenseArgs& a, hipStream_t s) {
  if (a.n_kv_tiles == 0) return hipSuccess;
  DkvArgs k{};
  k.q = (const uint16_t*)a.q; k.q_rope = (const uint16_t*)a.q_rope;
  k.k = (const uint16_t*)a.k; k.k_rope = (const uint16_t*)a.k_rope;
  k.v = (const uint16_t*)a.v; k.dy = (const uint16_t*)a.dy;
  k.lse2 = a.lse2; k.ndrow = a.ndrow;
  k.dk = (uint16_t*)a.dk; k.dk_rope = (uint16_t*)a.dk_rope; k.dv = (uint16_t*)a.dv;
  k.ds = (uint16_t*)a.ds;
  k.cu_q = a.cu_q; k.cu_kv = a.cu_kv; k.qt_base = a.qt_base; k.qt_blk = a.qt_blk; k.qt_kr = a.qt_kr;
  k.tiles = a.kv_tiles; k.split = a.kv_split; k.part = (float*)a.kv_part;
  k.n1 = a.n1; k.n2 = a.n2; k.G = a.G;
  k.lo_rel = a.mask_on ? a.lo_rel : -kBandInf; k.hi_rel = a.mask_on ? a.hi_rel : kBandInf; k.align = a.align;
  k.scale = a.scale; k.scale_log2e = a.scale_log2e;
  const bool ds = a.ds != nullptr;
  if (a.d_main == 128 && a.d_rope == 64 && a.d_v == 128)
    return launch_kv<128, 64, 128>(k, a.n_kv_tiles, ds, s);
  if (a.d_main == 128 && a.d_rope == 0 && a.d_v == 128)
    return launch_kv<128, 0, 128>(k, a.n_kv_tiles, ds, s);
  if (a.d_main == 64 && a.d_rope == 0 && a.d_v == 64) return launch_kv<64, 0, 64>(k, a.n_kv_tiles, ds, s);
  return hipErrorInvalidValue;
}


}  // namespace ab
