// Dense KV-major backward: dK and dV accumulated in registers, plus the dS tiles that
// the dQ product consumes (bf16 MFMA, fp32 accumulation).
//
// Page "aclnnFlashAttentionUnpaddingScoreGradV3", Formula section: dV = P^T dY,
// dK = dS^T Q / sqrt(d), dkRope = dS^T qRope / sqrt(d), with Q = [query, queryRope].
//
// One workgroup (4 waves) owns a 64-key tile of one sequence and KV head.  Query rows
// stream past in steps of 64 rows: the query tiles from the last one down to the diagonal
// (causal) or down to the first, each for the G query heads of the KV head in turn.
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
// Staging: a step's Q (query and queryRope parts), dY, lse2 and drow are loaded into
// registers one step ahead (while the current step computes) and written to one of two
// LDS stages at the end of the step.  (Global->LDS transfers were measured to slow the
// LDS reads of the compute phases in proportion to the bytes they move.)  Each part is a
// RowTile: every load instruction reads whole rows (full cache lines) and the chunk
// swizzle keeps the LDS writes and the row / column reads conflict free.
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

constexpr int kRows = 64;  // query rows per step, keys per workgroup
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
  int n1, n2, G;
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
// 8-byte store issued as inline assembly, so that the compiler does not hold back the
// next step's loads behind it.
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

// Per-lane addressing of one staged part (a RowTile of W chunks per row) for one wave.
//   loads: the wave fills 1 KB blocks i = w + 4k (k < W/4) of the part; lane l fills row
//              (w + 4k) RPI + l / W, slot l % W, i.e. reads chunk (l % W) ^ swz(row) --
//              the same chunk for every k, because 4 RPI rows is a multiple of 16.
//   row reads (A operands): rows 32rh + 16rt + l16, chunk 4s + g.
//   column reads (transposed, B operands): rows 32rh + 4g + jj (+16), chunk 2j + qq/2,
//              half qq&1.
template <int W>
struct PartLanes {
  using T = RowTile<W>;
  int row0;          // transfer row for k = 0
  uint32_t gchunk;   // byte offset of the chunk this lane reads within its row
  int rowA[W / 4];   // tile-relative byte offsets of the row reads (k-step s)
  int colB[W / 2];   // tile-relative byte offsets of the column reads (column tile j)
  __device__ __forceinline__ void init(int w, int lane, int rh) {
    const int l16 = lane & 15, g = lane >> 4, jj = l16 >> 2, qq = l16 & 3;
    row0 = w * T::RPI + lane / W;
    gchunk = 16u * (uint32_t)((lane % W) ^ T::swz(row0));
#pragma unroll
    for (int s = 0; s < W / 4; ++s) rowA[s] = T::off(32 * rh + l16, 4 * s + g);
#pragma unroll
    for (int j = 0; j < W / 2; ++j) colB[j] = T::off(32 * rh + 4 * g + jj, 2 * j + (qq >> 1)) + 8 * (qq & 1);
  }
};

template <int DM, int DR, int DV, bool DS>
__global__ __launch_bounds__(256, 1) void dense_kv_kernel(DkvArgs a) {
  constexpr int DQK = DM + DR;
  constexpr int KS = DQK / 32, VS = DV / 32, NQ = DQK / 16, NV = DV / 16;
  constexpr int KSM = DM / 32, NQM = DM / 16;  // k-steps / column tiles of the query part
  constexpr int WM = DM / 8, WR = DR > 0 ? DR / 8 : 8, WY = DV / 8;
  using TM = RowTile<WM>;
  using TR = RowTile<WR>;
  using TY = RowTile<WY>;
  constexpr int OQM = 0, OQR = TM::BYTES, OY = OQR + (DR > 0 ? TR::BYTES : 0);
  // stage: QM, QR, Y, lse2, drow, and two 256-byte slots the other waves' stat values land in
  constexpr int OL = OY + TY::BYTES, ORW = OL + 256, SB = ORW + 256 + 512;
  constexpr int NACC = 2 * (NQ + NV);
  constexpr int EPI = 2 * NACC * 1024 + 64 * (DQK + DV) * 2;           // epilogue buffers
  constexpr int SMEM = 2 * SB > EPI ? 2 * SB : EPI;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = w & 1, rh = w >> 1;
  const int l16 = lane & 15, g = lane >> 4;

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
      if (valid) x = ldg16(d < DM ? a.k + kr * DM + d : a.k_rope + kr * DR + (d - DM));
      Kf[t][s] = __builtin_bit_cast(bf16x8, x);
    }
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (valid) x = ldg16(a.v + kr * DV + 32 * s + 8 * g);
      Vf[t][s] = __builtin_bit_cast(bf16x8, x);
    }
  }
  // The K / V loads are the only vector-memory operations the compiler tracks; waiting for
  // them here keeps it from placing a full wait (which would also drain the transfers
  // issued ahead) inside the step loop, where the registers are first used.
  wait_vmcnt<0>();

  f32x4 dK[2][NQ], dV[2][NV];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) dK[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NV; ++n) dV[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  PartLanes<WM> pm;
  PartLanes<WR> pr;
  PartLanes<WY> py;
  pm.init(w, lane, rh);
  if constexpr (DR > 0) pr.init(w, lane, rh);
  py.init(w, lane, rh);

  // step st -> (query tile qt, head hg): query tiles walked from the last one down, the G
  // heads of a query tile back to back
  auto step_tile = [&](int st, int& hg, int& qt) {
    const int i = st / a.G;
    hg = st - i * a.G;
    qt = nqt - 1 - i;
  };

  const uint32_t smem_lds = lds_addr(smem);
  const uint32_t rs_m = (uint32_t)a.n1 * DM * 2, rs_r = (uint32_t)a.n1 * DR * 2, rs_y = (uint32_t)a.n1 * DV * 2;

  // Registers holding a stage on its way to LDS: W / 4 16-byte chunks per lane per part,
  // plus one lse2 (wave 0) or drow (wave 1) value per lane (row = lane).  Two sets, for
  // the stages one and two steps ahead.
  struct Regs {
    uint4 m[WM / 4], r[WR / 4], y[WY / 4];
    float st;
  };
  auto load_part = [&](auto wtag, const auto& pl, uint4* dst, const char* gtile, uint32_t rs, int nvalid) {
    constexpr int W = decltype(wtag)::value;
    constexpr int RPI = RowTile<W>::RPI;
#pragma unroll
    for (int k = 0; k < W / 4; ++k) {
      const int r = min(pl.row0 + 4 * RPI * k, nvalid - 1);
      dst[k] = ldg16(gtile + __umul24((uint32_t)r, rs) + pl.gchunk);
    }
  };
  auto load_stage = [&](int st, Regs& X) {
    int hg, qt;
    step_tile(st, hg, qt);
    const int nvalid = min(kRows, S1 - qt * kRows);
    const int64_t rh0 = (qs + (int64_t)qt * kRows) * a.n1 + kvh * a.G + hg;  // (first row) * n1 + h
    load_part(std::integral_constant<int, WM>{}, pm, X.m, reinterpret_cast<const char*>(a.q + rh0 * DM), rs_m, nvalid);
    if constexpr (DR > 0)
      load_part(std::integral_constant<int, WR>{}, pr, X.r, reinterpret_cast<const char*>(a.q_rope + rh0 * DR), rs_r,
                nvalid);
    load_part(std::integral_constant<int, WY>{}, py, X.y, reinterpret_cast<const char*>(a.dy + rh0 * DV), rs_y, nvalid);
    // every wave issues the same number of loads (waves 2, 3 read a value they drop)
    const int64_t lrow = rh0 + (int64_t)min(lane, nvalid - 1) * a.n1;
    X.st = w == 1 ? a.drow[lrow] : a.lse2[lrow];
  };
  auto write_stage = [&](int soff, const Regs& X) {
    const uint32_t stage = smem_lds + soff;
#pragma unroll
    for (int k = 0; k < WM / 4; ++k)
      lds_st16_at(stage + OQM + (w + 4 * k) * 1024 + 16 * lane, X.m[k]);
    if constexpr (DR > 0) {
#pragma unroll
      for (int k = 0; k < WR / 4; ++k)
        lds_st16_at(stage + OQR + (w + 4 * k) * 1024 + 16 * lane, X.r[k]);
    }
#pragma unroll
    for (int k = 0; k < WY / 4; ++k)
      lds_st16_at(stage + OY + (w + 4 * k) * 1024 + 16 * lane, X.y[k]);
    lds_st4_at(stage + OL + 256 * w + 4 * lane, X.st);  // waves 2, 3: unused slots
  };

  // dS of the previous step, stored at the start of the next one (see the loop)
  i16x4 dsv[2][2];
  uint16_t* dsp = nullptr;

  // One step.  Masks, all applied outside the MFMA stream: rows past the end of the
  // sequence get lse2 = +inf (P = 0); on the causal diagonal a short wave-uniform fix-up
  // zeroes P where key > row; keys past the end only matter for the stored dS, which is
  // zeroed for them (their dK / dV rows are never written).
  auto step_body = [&](int nvalid, bool diag, int soff) {
    const uint32_t stage = smem_lds + soff;
    const uint32_t statb = opaque(stage + OL + 4 * (32 * rh + 4 * g));  // lse2; drow at + 256

    f32x4 lse[2], dr[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      lse[rt] = lds_f32x4_at(statb + 64 * rt);
      dr[rt] = lds_f32x4_at(statb + 256 + 64 * rt);
    }
    if (nvalid < kRows) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) lse[rt][i] = 32 * rh + 16 * rt + 4 * g + i < nvalid ? lse[rt][i] : INFINITY;
    }
    // S = Q K^T, dP = dY V^T.  k-steps s < KSM read the query part, KSM <= s < KS the rope
    // part, the rest dY; the A fragments of a k-step (both row tiles) serve both key tiles
    // and are read PA k-steps ahead.
    constexpr int NS = KS + VS, PA = 3;
    auto afrag = [&](int s, int rt) -> bf16x8 {
      if (s < KSM) return lds_b128_at(stage + OQM + pm.rowA[s] + rt * 16 * TM::RB);
      if (s < KS) return lds_b128_at(stage + OQR + pr.rowA[s - KSM] + rt * 16 * TR::RB);
      return lds_b128_at(stage + OY + py.rowA[s - KS] + rt * 16 * TY::RB);
    };
    bf16x8 aring[PA][2];
#pragma unroll
    for (int i = 0; i < PA; ++i) { aring[i][0] = afrag(i, 0); aring[i][1] = afrag(i, 1); }
    f32x4 S[2][2], D[2][2];  // [key tile][row tile]
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 a0 = aring[s % PA][0], a1 = aring[s % PA][1];
      if (s + PA < NS) { aring[s % PA][0] = afrag(s + PA, 0); aring[s % PA][1] = afrag(s + PA, 1); }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (s < KS) {
          S[t][0] = mfma_16x16x32(a0, Kf[t][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : S[t][0]);
          S[t][1] = mfma_16x16x32(a1, Kf[t][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : S[t][1]);
        } else {
          D[t][0] = mfma_16x16x32(a0, Vf[t][s - KS], s == KS ? f32x4{0.f, 0.f, 0.f, 0.f} : D[t][0]);
          D[t][1] = mfma_16x16x32(a1, Vf[t][s - KS], s == KS ? f32x4{0.f, 0.f, 0.f, 0.f} : D[t][1]);
        }
      }
    }
    // schedule: the PA k-steps' reads first, then per k-step its 4 MFMAs and the reads of
    // the k-step PA ahead, so that each read has PA k-steps of MFMA work to land
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PA, 0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      if (s + PA < NS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    // P, then dS in place
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t][rt][i] = __builtin_amdgcn_exp2f(S[t][rt][i] * a.scale_log2e - lse[rt][i]);
    if (diag && kh == rh) {
      // keys 32kh + 16t + l16 against rows 32rh + 16rt + 4g + i: with kh == rh, tile pair
      // (t, rt) = (1, 0) lies wholly after the diagonal, (0, 1) wholly before it, and on
      // (0, 0) / (1, 1) the key lies after the row iff l16 - 4g > i
      const int dl = l16 - 4 * g;
      S[1][0] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool after = dl > i;
        S[0][0][i] = after ? 0.f : S[0][0][i];
        S[1][1][i] = after ? 0.f : S[1][1][i];
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) D[t][rt][i] = S[t][rt][i] * (D[t][rt][i] - dr[rt][i]);
    // dV += P^T dY, dK += dS^T Q.  Items j < NV: dY columns 16j.. (dV); then the query and
    // rope columns (dK).  Each column fragment (two transposed reads) serves both key tiles
    // and is read PD items ahead of its MFMAs.
    bf16x8 pa[2], da[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      pa[t] = pack8(S[t][0], S[t][1]);
      da[t] = pack8(D[t][0], D[t][1]);
      const i16x8 dv8 = __builtin_bit_cast(i16x8, da[t]);
      dsv[t][0] = i16x4{dv8[0], dv8[1], dv8[2], dv8[3]};
      dsv[t][1] = i16x4{dv8[4], dv8[5], dv8[6], dv8[7]};
      if (nk < kRows && 32 * kh + 16 * t + l16 >= nk) dsv[t][0] = dsv[t][1] = i16x4{0, 0, 0, 0};
    }
    auto colfrag = [&](int j) -> bf16x8 {
      uint32_t o, second;
      if (j < NV) { o = stage + OY + py.colB[j]; second = 16 * TY::RB; }
      else if (j < NV + NQM) { o = stage + OQM + pm.colB[j - NV]; second = 16 * TM::RB; }
      else { o = stage + OQR + pr.colB[j - NV - NQM]; second = 16 * TR::RB; }
      return join8(lds_tr16_at(o), lds_tr16_at(o + second));
    };
    constexpr int NJ = NV + NQ, PD = 4;
    bf16x8 ring[PD];
#pragma unroll
    for (int i = 0; i < PD; ++i) ring[i] = colfrag(i);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const bf16x8 bj = ring[j % PD];
      if (j + PD < NJ) ring[j % PD] = colfrag(j + PD);
      if (j < NV) {
        dV[0][j] = mfma_16x16x32(pa[0], bj, dV[0][j]);
        dV[1][j] = mfma_16x16x32(pa[1], bj, dV[1][j]);
      } else {
        dK[0][j - NV] = mfma_16x16x32(da[0], bj, dK[0][j - NV]);
        dK[1][j - NV] = mfma_16x16x32(da[1], bj, dK[1][j - NV]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PD, 1);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
      if (j + PD < NJ) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
  };

  // this lane's place in the dS^T block [64 keys][64 rows] of step st's (query tile, key
  // tile kt0, head)
  auto ds_ptr = [&](int st) -> uint16_t* {
    int hg, qt;
    step_tile(st, hg, qt);
    const int64_t blk = blk0 + (a.causal ? (int64_t)qt * (qt + 1) / 2 + kt0 : (int64_t)qt * nkt + kt0);
    return a.ds + (blk * a.n1 + kvh * a.G + hg) * (int64_t)(kRows * kRows) + (32 * kh + l16) * kRows + 32 * rh + 4 * g;
  };
  auto step = [&](int st, int soff) {
    int hg, qt;
    step_tile(st, hg, qt);
    const int nvalid = min(kRows, S1 - qt * kRows);
    const bool diag = a.causal && qt == kt0;
    if constexpr (DS) dsp = ds_ptr(st);
    if (diag && kh > rh) {  // every key of this wave lies after every row: P = dS = 0
#pragma unroll
      for (int t = 0; t < 2; ++t) dsv[t][0] = dsv[t][1] = i16x4{0, 0, 0, 0};
      return;
    }
    step_body(nvalid, diag, soff);
  };

  auto store_ds = [&]() {
    // rows 32rh + 4g + (0..3) and + 16; keys 32kh + 16t + l16
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      *reinterpret_cast<i16x4*>(dsp + 16 * t * kRows) = dsv[t][0];
      *reinterpret_cast<i16x4*>(dsp + 16 * t * kRows + 16) = dsv[t][1];
    }
  };

  // Iteration st: barrier (stage st is written; stage st+1 is no longer read), store the
  // dS of step st-1, compute step st, write the registers holding stage st+1 into LDS and
  // reload them with stage st+3.  Stage k's loads are issued at the end of iteration k-3
  // and wait at the end of iteration k-1: two steps to arrive.  Iterations alternate
  // between the two register sets (the loop is unrolled by two).
  // The memory operations of every iteration are the same: the dS store of the previous
  // step (in iteration 0 and before it: zeros into step 0's block, which step 0's own
  // store overwrites later), the wait for one register set, the loads into it (past the
  // last step they repeat the last stage, which is never written to LDS).  So the waits
  // the compiler places before each write_stage count exactly the newer operations and
  // leave the other set in flight.
  Regs ra, rb;
  if (nsteps > 0) {
    if constexpr (DS) {
      dsp = ds_ptr(0);
#pragma unroll
      for (int t = 0; t < 2; ++t) dsv[t][0] = dsv[t][1] = i16x4{0, 0, 0, 0};
    }
    load_stage(0, ra);
    write_stage(0, ra);
    load_stage(min(1, nsteps - 1), ra);
    if constexpr (DS) store_ds();
    load_stage(min(2, nsteps - 1), rb);
  }
  auto iteration = [&](int st, Regs& X) {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    barrier_no_vm_wait();
    if constexpr (DS) store_ds();
    step(st, (st & 1) * SB);
    if (st + 1 < nsteps) write_stage((~st & 1) * SB, X);
    load_stage(min(st + 3, nsteps - 1), X);
  };
  int st = 0;
  for (; st + 1 < nsteps; st += 2) {
    iteration(st, ra);
    iteration(st + 1, rb);
  }
  if (st < nsteps) iteration(st, ra);
  if (DS && nsteps > 0) store_ds();

  // ---- epilogue: sum the two row halves, bf16 through LDS, 16-byte stores ------------
  __syncthreads();
  // partials of the rh = 1 waves: [kh][index][lane] as f32x4 (conflict-free)
  f32x4* part = reinterpret_cast<f32x4*>(smem);
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
  // output tiles, row-major: dK [64 keys][DQK], dV [64 keys][DV]
  uint16_t* Ko = reinterpret_cast<uint16_t*>(smem + 2 * NACC * 1024);
  uint16_t* Vo = Ko + 64 * DQK;
  if (rh == 0) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        const f32x4 o = part[(kh * NACC + t * (NQ + NV) + n) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Ko[(32 * kh + 16 * t + 4 * g + i) * DQK + 16 * n + l16] = f2bf((dK[t][n][i] + o[i]) * a.scale);
      }
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        const f32x4 o = part[(kh * NACC + t * (NQ + NV) + NQ + n) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) Vo[(32 * kh + 16 * t + 4 * g + i) * DV + 16 * n + l16] = f2bf(dV[t][n][i] + o[i]);
      }
    }
  }
  __syncthreads();
  constexpr int QCH = DQK / 8, YCH = DV / 8;
  for (int idx = tid; idx < kRows * QCH; idx += 256) {
    const int r = idx / QCH, c = idx - r * QCH, d = 8 * c;
    if (r < nk) {
      const int64_t kr = (k0 + r) * a.n2 + kvh;
      uint16_t* dst = d < DM ? a.dk + kr * DM + d : a.dk_rope + kr * DR + (d - DM);
      sts16(dst, *reinterpret_cast<const uint4*>(Ko + r * DQK + d));
    }
  }
  for (int idx = tid; idx < kRows * YCH; idx += 256) {
    const int r = idx / YCH, c = idx - r * YCH;
    if (r < nk) sts16(a.dv + ((k0 + r) * a.n2 + kvh) * DV + 8 * c, *reinterpret_cast<const uint4*>(Vo + r * DV + 8 * c));
  }
}

template <int DM, int DR, int DV>
hipError_t launch_kv(const DkvArgs& k, dim3 grid, bool ds, hipStream_t s) {
  if (ds) hipLaunchKernelGGL((dense_kv_kernel<DM, DR, DV, true>), grid, dim3(256), 0, s, k);
  else hipLaunchKernelGGL((dense_kv_kernel<DM, DR, DV, false>), grid, dim3(256), 0, s, k);
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
  k.lse2 = a.lse2; k.drow = a.drow;
  k.dk = (uint16_t*)a.dk; k.dk_rope = (uint16_t*)a.dk_rope; k.dv = (uint16_t*)a.dv;
  k.ds = (uint16_t*)a.ds;
  k.cu_q = a.cu_q; k.cu_kv = a.cu_kv; k.ds_base = a.ds_base; k.tiles = a.kv_tiles;
  k.n1 = a.n1; k.n2 = a.n2; k.G = a.G;
  k.causal = a.causal; k.scale = a.scale; k.scale_log2e = a.scale_log2e;
  const dim3 grid(a.n_kv_tiles);
  const bool ds = a.ds != nullptr;
  if (a.d_main == 128 && a.d_rope == 64 && a.d_v == 128) return launch_kv<128, 64, 128>(k, grid, ds, s);
  if (a.d_main == 128 && a.d_rope == 0 && a.d_v == 128) return launch_kv<128, 0, 128>(k, grid, ds, s);
  if (a.d_main == 64 && a.d_rope == 0 && a.d_v == 64) return launch_kv<64, 0, 64>(k, grid, ds, s);
  return hipErrorInvalidValue;
}

}  // namespace ab
