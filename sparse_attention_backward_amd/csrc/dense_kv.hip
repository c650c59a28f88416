// Dense KV-major backward: dK and dV accumulated in registers, plus the dS tiles that
// the dQ product consumes (bf16 MFMA, fp32 accumulation).
//
// Page "aclnnFlashAttentionUnpaddingScoreGradV3", Formula section: dV = P^T dY,
// dK = dS^T Q / sqrt(d), dkRope = dS^T qRope / sqrt(d), with Q = [query, queryRope].
//
// One workgroup (4 waves) owns a 128-key tile of one sequence and KV head, and a range of
// its query tiles.  Query rows stream past in steps of 64 rows: the query tiles of the
// range from the last one down, each for the G query heads of the KV head in turn.
// Walking every key tile's list from the same end keeps the workgroups of one
// (sequence, KV head) on the same query tile at the same time, so their row loads share
// the L2.  A step's rows are loaded once for 128 keys (half the load and LDS-write
// traffic per flop of a 64-key tile, and half the barriers).
//
// Wave w owns keys 32w .. +31 of the tile (K and V resident in registers as MFMA B
// operands) and takes the two 32-row halves of every step in turn.  Per half (32 rows x
// 32 keys):
//   S = Q K^T, dP = dY V^T       A operands: Q / dY rows from LDS (16-byte reads)
//   P = exp2(S*scale*log2e - lse2), dS = P (dP - drow)   (masks: causal diagonal,
//                                 ragged query tail, ragged key tail)
//   dV += P^T dY, dK += dS^T Q   A operands: the P / dS C tiles repacked in registers;
//                                 B operands: dY / Q columns (ds_read_b64_tr_b16)
//   dS^T -> workspace (bf16), one 64 x 64 block per (query tile, 64-key tile, head)
// Causal: a wave's 32-key block against a 32-row block is skipped when it lies wholly
// after the rows, masked on the diagonal, and complete otherwise.
//
// Key tiles with many query tiles are split into ranges (so that no workgroup runs far
// longer than the average): each range leaves its fp32 dK / dV in a partial slot, in
// register order, and dense_kv_combine_kernel adds the ranges of a tile in range order.
// Every output row has one writer: no atomics, deterministic.
//
// Staging: a step's Q (query and queryRope parts), dY, lse2 and drow are loaded into
// registers two steps ahead (two register sets) and written to one of two LDS stages at
// the end of the step before.  Each part is a RowTile: every load instruction reads whole
// rows (full cache lines) and the chunk swizzle keeps the LDS writes and the row / column
// reads conflict free.
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
  const float* lse2; const float* drow;
  uint16_t* dk; uint16_t* dk_rope; uint16_t* dv;
  uint16_t* ds;               // [block][head][64 keys][64 rows] bf16 (dS transposed)
  const int64_t* cu_q; const int64_t* cu_kv;
  const int64_t* ds_base;     // [B + 1] (query tile, 64-key tile) blocks before each sequence
  const int32_t* tiles;       // [n][6] (sequence, 128-key tile, KV head, first / end query tile,
                              // partial slot or -1); sequence < 0: idle slot
  const int32_t* split;       // [n][5] (sequence, 128-key tile, KV head, first slot, parts)
  float* part;                // fp32 partials, kDenseKvPartBytes per slot
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
//   row reads (A operands): rows 16rt + l16, chunk 4s + g (+32 rows for the second half).
//   column reads (transposed, B operands): rows 4g + jj (+16), chunk 2j + qq/2, half qq&1
//              (+32 rows for the second half).
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

// dK (scaled) / dV of this wave's 32 keys from the accumulators to bf16 rows through LDS
// (Ko [128][DQK], Vo [128][DV] at smem), then 16-byte stores of the rows < nk.
template <int DM, int DR, int DV>
__device__ __forceinline__ void store_dkdv(const DkvArgs& a, char* smem, const f32x4 (&dK)[2][(DM + DR) / 16],
                                           const f32x4 (&dV)[2][DV / 16], int w, int lane, int64_t k0, int nk,
                                           int kvh) {
  constexpr int DQK = DM + DR, NQ = DQK / 16, NV = DV / 16;
  const int l16 = lane & 15, g = lane >> 4;
  uint16_t* Ko = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vo = Ko + kKeys * DQK;
  __syncthreads();  // LDS free
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int n = 0; n < NQ; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) Ko[(32 * w + 16 * t + 4 * g + i) * DQK + 16 * n + l16] = f2bf(dK[t][n][i] * a.scale);
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) Vo[(32 * w + 16 * t + 4 * g + i) * DV + 16 * n + l16] = f2bf(dV[t][n][i]);
  }
  __syncthreads();
  constexpr int QCH = DQK / 8, YCH = DV / 8;
  const int tid = 64 * w + lane;
  for (int idx = tid; idx < kKeys * QCH; idx += 256) {
    const int r = idx / QCH, c = idx - r * QCH, d = 8 * c;
    if (r < nk) {
      const int64_t kr = (k0 + r) * a.n2 + kvh;
      uint16_t* dst = d < DM ? a.dk + kr * DM + d : a.dk_rope + kr * DR + (d - DM);
      sts16(dst, *reinterpret_cast<const uint4*>(Ko + r * DQK + d));
    }
  }
  for (int idx = tid; idx < kKeys * YCH; idx += 256) {
    const int r = idx / YCH, c = idx - r * YCH;
    if (r < nk) sts16(a.dv + ((k0 + r) * a.n2 + kvh) * DV + 8 * c, *reinterpret_cast<const uint4*>(Vo + r * DV + 8 * c));
  }
}

template <int DM, int DR, int DV, bool DS>
__global__ __launch_bounds__(256, 1) void dense_kv_kernel(DkvArgs a) {
  constexpr int DQK = DM + DR;
  constexpr int KS = DQK / 32, VS = DV / 32, NQ = DQK / 16, NV = DV / 16;
  constexpr int KSM = DM / 32, NQM = DM / 16;  // k-steps / column tiles of the query part
  constexpr int WM = DM / 8, WR = DR > 0 ? DR / 8 : 8, WY = DV / 8;
  using TM = RowTile<WM>;
  using TR = RowTile<WR>;
  using TY = RowTile<WY>;
  // stage: QM, QR, Y, lse2, drow, and two 256-byte slots the other waves' stat values land in
  constexpr int OQM = 0, OQR = TM::BYTES, OY = OQR + (DR > 0 ? TR::BYTES : 0);
  constexpr int OL = OY + TY::BYTES, ORW = OL + 256, SB = ORW + 256 + 512;
  constexpr int EPI = kKeys * (DQK + DV) * 2;  // epilogue: bf16 output tiles
  constexpr int SMEM = 2 * SB > EPI ? 2 * SB : EPI;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  static_assert(2 * (NQ + NV) * 16 * 256 <= kDenseKvPartBytes, "partial slot size");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int64_t blk0 = a.ds_base[b];
  const int kb = 4 * kt0 + w;          // this wave's 32-key block
  const int kt64 = 2 * kt0 + (w >> 1);  // its 64-key tile (dS block column)
  const bool idle = 32 * w >= nk;       // every key of this wave lies past the sequence

  // ---- resident keys: K and V as MFMA B operands ------------------------------------
  bf16x8 Kf[2][KS], Vf[2][VS];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = 32 * w + 16 * t + l16;
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
  // them here keeps it from placing a full wait inside the step loop.
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
  pm.init(w, lane, 0);
  if constexpr (DR > 0) pr.init(w, lane, 0);
  py.init(w, lane, 0);

  // step st -> (query tile qt, head hg): the range's query tiles from the last one down,
  // the G heads of a query tile back to back
  auto step_tile = [&](int st, int& hg, int& qt) {
    const int i = st / a.G;
    hg = st - i * a.G;
    qt = qb - 1 - i;
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


  // One half step: rows 32 hi .. +31 of step st.  Masks, all applied outside the MFMA
  // stream: rows past the end of the sequence get lse2 = +inf (P = 0); on the causal
  // diagonal a short wave-uniform fix-up zeroes P where key > row; keys past the end only
  // matter for the stored dS, which is zeroed for them (their dK / dV rows are never
  // written).
  auto half_step = [&](int st, uint32_t stage, auto hic) {
    constexpr int hi = decltype(hic)::value;
    int hg, qt;
    step_tile(st, hg, qt);
    const int rb = 2 * qt + hi;  // this half's 32-row block
    uint16_t* dsp = nullptr;
    if constexpr (DS) {
      if (kt64 < nkt64 && (!a.causal || kt64 <= qt)) {  // the block exists
        const int64_t blk = blk0 + (a.causal ? (int64_t)qt * (qt + 1) / 2 + kt64 : (int64_t)qt * nkt64 + kt64);
        dsp = a.ds + (blk * a.n1 + kvh * a.G + hg) * (int64_t)(kRows * kRows) + (32 * (w & 1) + l16) * kRows +
              32 * hi + 4 * g;
      }
    }
    // a wave with no key in the sequence, or with every key after every row, contributes
    // nothing and only writes zeros to its part of an existing dS block
    const bool active = !idle && !(a.causal && kb > rb);
    bf16x8 da[2] = {bf16x8{}, bf16x8{}};
    if (active) {
    const bool diag = a.causal && kb == rb;
    const int nvalid = min(kRows, S1 - qt * kRows);
    const uint32_t bm = stage + OQM + hi * 32 * TM::RB, br = stage + OQR + hi * 32 * TR::RB;
    const uint32_t by = stage + OY + hi * 32 * TY::RB;
    const uint32_t statb = opaque(stage + OL + 4 * (32 * hi + 4 * g));  // lse2; drow at + 256

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
        for (int i = 0; i < 4; ++i) lse[rt][i] = 32 * hi + 16 * rt + 4 * g + i < nvalid ? lse[rt][i] : INFINITY;
    }
    // S = Q K^T, dP = dY V^T.  k-steps s < KSM read the query part, KSM <= s < KS the rope
    // part, the rest dY; the A fragments of a k-step (both row tiles) serve both key tiles
    // and are read PA k-steps ahead.
    constexpr int NS = KS + VS, PA = 3;
    auto afrag = [&](int s, int rt) -> bf16x8 {
      if (s < KSM) return lds_b128_at(bm + pm.rowA[s] + rt * 16 * TM::RB);
      if (s < KS) return lds_b128_at(br + pr.rowA[s - KSM] + rt * 16 * TR::RB);
      return lds_b128_at(by + py.rowA[s - KS] + rt * 16 * TY::RB);
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
    if (diag) {
      // keys 32kb + 16t + l16 against rows 32kb + 16rt + 4g + i: tile pair (t, rt) = (1, 0)
      // lies wholly after the diagonal, (0, 1) wholly before it, and on (0, 0) / (1, 1)
      // the key lies after the row iff l16 - 4g > i
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
    bf16x8 pa[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      pa[t] = pack8(S[t][0], S[t][1]);
      da[t] = pack8(D[t][0], D[t][1]);
    }
    auto colfrag = [&](int j) -> bf16x8 {
      uint32_t o, second;
      if (j < NV) { o = by + py.colB[j]; second = 16 * TY::RB; }
      else if (j < NV + NQM) { o = bm + pm.colB[j - NV]; second = 16 * TM::RB; }
      else { o = br + pr.colB[j - NV - NQM]; second = 16 * TR::RB; }
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
    }  // active
    if constexpr (DS) {
      // dS^T rows (keys) 32(w&1) + 16t + l16 of the 64-key tile, columns (query rows)
      // 32hi + 4g + (0..3) and + 16
      if (dsp != nullptr)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const i16x8 d8 = __builtin_bit_cast(i16x8, da[t]);
        i16x4 lo = i16x4{d8[0], d8[1], d8[2], d8[3]}, hv = i16x4{d8[4], d8[5], d8[6], d8[7]};
        if (nk < kKeys && 32 * w + 16 * t + l16 >= nk) lo = hv = i16x4{0, 0, 0, 0};
        *reinterpret_cast<i16x4*>(dsp + 16 * t * kRows) = lo;
        *reinterpret_cast<i16x4*>(dsp + 16 * t * kRows + 16) = hv;
      }
    }
  };

  // Iteration st: barrier (stage st is written; stage st+1 is no longer read), the two
  // half steps of step st (each storing its dS^T), then the registers holding stage st+1
  // go to LDS and are reloaded with stage st+3.  Stage k's loads are issued at the end of
  // iteration k-3 and wait at the end of iteration k-1: two steps to arrive.  Iterations
  // alternate between the two register sets (the loop is unrolled by two).  Past the last
  // step the loads repeat the last stage (never written to LDS), so that every iteration
  // issues the same loads.
  Regs ra, rb;
  if (nsteps > 0) {
    load_stage(0, ra);
    write_stage(0, ra);
    load_stage(min(1, nsteps - 1), ra);
    load_stage(min(2, nsteps - 1), rb);
  }
  auto iteration = [&](int st, Regs& X) {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    barrier_no_vm_wait();
    const uint32_t stage = smem_lds + (st & 1) * SB;
    half_step(st, stage, std::integral_constant<int, 0>{});
    half_step(st, stage, std::integral_constant<int, 1>{});
    if (st + 1 < nsteps) write_stage((~st & 1) * SB, X);
    load_stage(min(st + 3, nsteps - 1), X);
  };
  int st = 0;
  for (; st + 1 < nsteps; st += 2) {
    iteration(st, ra);
    iteration(st + 1, rb);
  }
  if (st < nsteps) iteration(st, ra);

  // ---- epilogue --------------------------------------------------------------------------
  if (slot < 0) {
    store_dkdv<DM, DR, DV>(a, smem, dK, dV, w, lane, k0, nk, kvh);
  } else {
    // fp32 partial in register order: [wave][register][lane] f32x4, coalesced 16-byte stores
    f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<char*>(a.part) + (size_t)slot * kDenseKvPartBytes) +
                 w * (2 * (NQ + NV)) * 64 + lane;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int n = 0; n < NQ; ++n) dst[(t * (NQ + NV) + n) * 64] = dK[t][n];
#pragma unroll
      for (int n = 0; n < NV; ++n) dst[(t * (NQ + NV) + NQ + n) * 64] = dV[t][n];
    }
  }
}

// dK / dV of a split key tile: the partials of its query ranges added in range order.
template <int DM, int DR, int DV>
__global__ __launch_bounds__(256, 1) void dense_kv_combine_kernel(DkvArgs a) {
  constexpr int DQK = DM + DR, NQ = DQK / 16, NV = DV / 16;
  __shared__ __attribute__((aligned(1024))) char smem[kKeys * (DQK + DV) * 2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t* sp = a.split + 5 * blockIdx.x;
  const int b = sp[0], kt0 = sp[1], kvh = sp[2], slot0 = sp[3], parts = sp[4];
  const int64_t ks = a.cu_kv[b];
  const int S2 = (int)(a.cu_kv[b + 1] - ks);
  const int64_t k0 = ks + (int64_t)kt0 * kKeys;
  const int nk = min(kKeys, S2 - kt0 * kKeys);
  f32x4 dK[2][NQ], dV[2][NV];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) dK[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NV; ++n) dV[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int p = 0; p < parts; ++p) {
    const f32x4* src = reinterpret_cast<const f32x4*>(reinterpret_cast<const char*>(a.part) +
                                                      (size_t)(slot0 + p) * kDenseKvPartBytes) +
                       w * (2 * (NQ + NV)) * 64 + lane;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int n = 0; n < NQ; ++n) dK[t][n] += src[(t * (NQ + NV) + n) * 64];
#pragma unroll
      for (int n = 0; n < NV; ++n) dV[t][n] += src[(t * (NQ + NV) + NQ + n) * 64];
    }
  }
  store_dkdv<DM, DR, DV>(a, smem, dK, dV, w, lane, k0, nk, kvh);
}

template <int DM, int DR, int DV>
hipError_t launch_kv(const DkvArgs& k, int n_tiles, int n_split, bool ds, bool combine, hipStream_t s) {
  if (!combine && n_tiles > 0) {
    if (ds) hipLaunchKernelGGL((dense_kv_kernel<DM, DR, DV, true>), dim3(n_tiles), dim3(256), 0, s, k);
    else hipLaunchKernelGGL((dense_kv_kernel<DM, DR, DV, false>), dim3(n_tiles), dim3(256), 0, s, k);
  }
  if (combine && n_split > 0)
    hipLaunchKernelGGL((dense_kv_combine_kernel<DM, DR, DV>), dim3(n_split), dim3(256), 0, s, k);
  return hipGetLastError();
}

}  // namespace

bool dense_bf16_supported(int d_main, int d_rope, int d_v) {
  return (d_main == 128 && d_rope == 64 && d_v == 128) || (d_main == 128 && d_rope == 0 && d_v == 128) ||
         (d_main == 64 && d_rope == 0 && d_v == 64);
}

static hipError_t launch_dense_kv_any(const DenseArgs& a, bool combine, hipStream_t s) {
  if (a.n_kv_tiles == 0) return hipSuccess;
  DkvArgs k{};
  k.q = (const uint16_t*)a.q; k.q_rope = (const uint16_t*)a.q_rope;
  k.k = (const uint16_t*)a.k; k.k_rope = (const uint16_t*)a.k_rope;
  k.v = (const uint16_t*)a.v; k.dy = (const uint16_t*)a.dy;
  k.lse2 = a.lse2; k.drow = a.drow;
  k.dk = (uint16_t*)a.dk; k.dk_rope = (uint16_t*)a.dk_rope; k.dv = (uint16_t*)a.dv;
  k.ds = (uint16_t*)a.ds;
  k.cu_q = a.cu_q; k.cu_kv = a.cu_kv; k.ds_base = a.ds_base;
  k.tiles = a.kv_tiles; k.split = a.kv_split; k.part = (float*)a.kv_part;
  k.n1 = a.n1; k.n2 = a.n2; k.G = a.G;
  k.causal = a.causal; k.scale = a.scale; k.scale_log2e = a.scale_log2e;
  const bool ds = a.ds != nullptr;
  if (a.d_main == 128 && a.d_rope == 64 && a.d_v == 128)
    return launch_kv<128, 64, 128>(k, a.n_kv_tiles, a.n_kv_split, ds, combine, s);
  if (a.d_main == 128 && a.d_rope == 0 && a.d_v == 128)
    return launch_kv<128, 0, 128>(k, a.n_kv_tiles, a.n_kv_split, ds, combine, s);
  if (a.d_main == 64 && a.d_rope == 0 && a.d_v == 64) return launch_kv<64, 0, 64>(k, a.n_kv_tiles, a.n_kv_split, ds, combine, s);
  return hipErrorInvalidValue;
}

hipError_t launch_dense_kv_bf16(const DenseArgs& a, hipStream_t s) { return launch_dense_kv_any(a, false, s); }

hipError_t launch_dense_kv_combine(const DenseArgs& a, hipStream_t s) { return launch_dense_kv_any(a, true, s); }

}  // namespace ab
