// Dense dQ from the stored dS tiles: dQ = scale * dS K (bf16 MFMA, fp32 accumulation).
//
// Page "aclnnFlashAttentionUnpaddingScoreGradV3", Formula section: dQ = dS K / sqrt(d),
// dqRope = dS kRope / sqrt(d), with K = [key, keyRope].  dS itself comes from the KV-major
// kernel, which leaves one transposed 64 x 64 bf16 block per (query tile, key tile, head)
// in the workspace; this kernel is then a plain product, with no recomputation of S or dP.
//
// One workgroup (8 waves) owns a 64-row query tile of HP query heads that share a KV head
// (all G heads, in passes of HP).  Per key tile it stages the K tile (key and keyRope
// parts) and the HP dS^T blocks in LDS through global->LDS transfers and accumulates
// dQ += dS K.  The K tile is re-read by every query tile of its KV head and mostly comes
// from L2, so two K stages (one tile ahead) suffice; the dS^T blocks are read once from
// HBM, so they rotate through three stages, issued two tiles ahead.  Each wave owns one
// head, a group of rows and one half of the features.  Both operands are read with
// ds_read_b64_tr_b16: the contraction runs over keys, which are the rows of both staged
// tiles (RowTile layout: whole-row transfers, conflict-free column reads).  Keys are
// taken in the order {4g + j, 16 + 4g + j} on both sides.  Fixed loop order, no atomics:
// deterministic.
//
// The same launch also finishes the key tiles that the KV-major kernel split into query
// ranges (both depend only on that kernel): its first n_split workgroups each add the fp32
// partials of one split key tile in range order and write its dK (scaled) and dV rows.
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

constexpr int kT = 64;  // rows per query tile, keys per key tile
typedef __attribute__((address_space(3))) void lds_void;

struct DqArgs {
  const uint16_t* k; const uint16_t* k_rope;
  const uint16_t* ds;           // [block][head][64 keys][64 rows]
  uint16_t* dq; uint16_t* dq_rope;
  const int64_t* cu_q; const int64_t* cu_kv;
  const int32_t* qt_base;       // [B + 1] query tiles before each sequence
  const int64_t* qt_blk;        // first stored block of each query tile
  const int32_t* qt_kr;         // [query tiles][2] its 64-key tiles [lo, hi)
  const int32_t* tiles;         // [n][2] (sequence, query tile)
  int n1, n2, G;
  float scale;
  int n_q_tiles;                // workgroups: n_split, then (query tile, KV head), KV head fastest
  // split key tiles of the KV-major kernel
  const int32_t* split;         // [n_split][5] (sequence, 128-key tile, KV head, first slot, parts)
  const float* part;            // fp32 partials, kDenseKvPartBytes per slot, [pair][register][lane]
  uint16_t* dk; uint16_t* dk_rope; uint16_t* dv;
  int n_split;
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void barrier_no_vm_wait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* lds) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds);
}

template <int MOFF>
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               ::"v"(src), "s"(lds), "i"(MOFF) : "memory", "m0", "scc");
}
// the same with the non-temporal hint, for data read once (dS): it does not displace the
// K tiles that later query tiles re-read from L2
template <int MOFF>
__device__ __forceinline__ void dma16_nt(const void* src, uint32_t lds) {
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               ::"v"(src), "s"(lds), "i"(MOFF) : "memory", "m0", "scc");
}

template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

// Per-lane addressing of one staged part (RowTile of W chunks, 64 key rows) for wave w:
// transfer row / chunk (as in the KV-major kernel) and the transposed column reads
// (keys 4g + jj (+16), chunk 2j + qq/2, half qq&1).
template <int W>
struct KeyPartLanes {
  using T = RowTile<W>;
  int row0;
  uint32_t gchunk;
  int colB[W / 2];
  __device__ __forceinline__ void init(int w, int lane) {
    const int l16 = lane & 15, g = lane >> 4, jj = l16 >> 2, qq = l16 & 3;
    row0 = w * T::RPI + lane / W;
    gchunk = 16u * (uint32_t)((lane % W) ^ T::swz(row0));
#pragma unroll
    for (int j = 0; j < W / 2; ++j) colB[j] = T::off(4 * g + jj, 2 * j + (qq >> 1)) + 8 * (qq & 1);
  }
};

// dK / dV of split key tile sidx: the partials of its ranges added in range order (waves
// 0-3: dK of key pair w, waves 4-7: dV of key pair w - 4), then bf16 rows through LDS
// (dK [128][DQK] scaled, dV [128][DV]) and 16-byte stores of rows < nk.
template <int DM, int DR, int DV>
__device__ __forceinline__ void combine_split_tile(const DqArgs& a, int sidx, char* smem) {
  constexpr int DQK = DM + DR, NQ = DQK / 16, NV = DV / 16, KEYS = kDenseKeyTile;
  static_assert(KEYS * (DQK + DV) * 2 <= 160 * 1024, "output tiles");
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pr = w & 3, l16 = lane & 15, g = lane >> 4;
  const int32_t* sp = a.split + 5 * sidx;
  const int b = sp[0], kt0 = sp[1], kvh = sp[2], slot0 = sp[3], parts = sp[4];
  const int64_t ks = a.cu_kv[b];
  const int S2 = (int)(a.cu_kv[b + 1] - ks);
  const int64_t k0 = ks + (int64_t)kt0 * KEYS;
  const int nk = min(KEYS, S2 - kt0 * KEYS);
  uint16_t* Ko = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vo = Ko + KEYS * DQK;
  // one kind of accumulator per wave: N tiles at register offset R of the pair's slot region
  auto sum_parts = [&](auto nc, auto rc, uint16_t* tile, int D, float sc) {
    constexpr int N = decltype(nc)::value, R = decltype(rc)::value;
    f32x4 acc[2][N];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int n = 0; n < N; ++n) acc[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < parts; ++q) {
      const f32x4* src = reinterpret_cast<const f32x4*>(reinterpret_cast<const char*>(a.part) +
                                                        (size_t)(slot0 + q) * kDenseKvPartBytes) +
                         pr * (2 * (NQ + NV)) * 64 + lane;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int n = 0; n < N; ++n) acc[t][n] += src[(t * (NQ + NV) + R + n) * 64];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < N; ++n) tile[(32 * pr + 16 * t + 4 * g + i) * D + 16 * n + l16] = f2bf(acc[t][n][i] * sc);
  };
  if (w < 4) sum_parts(std::integral_constant<int, NQ>{}, std::integral_constant<int, 0>{}, Ko, DQK, a.scale);
  else sum_parts(std::integral_constant<int, NV>{}, std::integral_constant<int, NQ>{}, Vo, DV, 1.f);
  __syncthreads();
  constexpr int QCH = DQK / 8, YCH = DV / 8;
  for (int idx = tid; idx < KEYS * QCH; idx += 512) {
    const int r = idx / QCH, c = idx - r * QCH, d = 8 * c;
    if (r < nk) {
      const int64_t kr = (k0 + r) * a.n2 + kvh;
      uint16_t* dst = d < DM ? a.dk + kr * DM + d : a.dk_rope + kr * DR + (d - DM);
      sts16(dst, *reinterpret_cast<const uint4*>(Ko + r * DQK + d));
    }
  }
  for (int idx = tid; idx < KEYS * YCH; idx += 512) {
    const int r = idx / YCH, c = idx - r * YCH;
    if (r < nk) sts16(a.dv + ((k0 + r) * a.n2 + kvh) * DV + 8 * c, *reinterpret_cast<const uint4*>(Vo + r * DV + 8 * c));
  }
}

// 8 waves: WPH = 8 / HP waves per head; within a head, wave (rs, fh) takes query rows
// 16 RT rs .. (RT = HP row tiles of 16, R = 4 / HP row groups) and feature half fh.  Each
// dS^T column fragment (A operand) serves the NF feature tiles of the wave, each K column
// fragment (B operand) its RT row tiles.
template <int DM, int DR, int HP>
__global__ __launch_bounds__(512, 1) void dense_dq_ds_kernel(DqArgs a) {
  constexpr int DQK = DM + DR;
  constexpr int NQ = DQK / 16, NF = NQ / 2, NQM = DM / 16;  // feature tiles: all / per wave / key part
  constexpr int WM = DM / 8, WR = DR > 0 ? DR / 8 : 8;
  constexpr int WPH = 8 / HP, RT = HP;                     // waves per head, row tiles per wave
  using TM = RowTile<WM>;
  using TR = RowTile<WR>;
  using TD = RowTile<8>;                                     // dS^T block: 64 keys x 64 rows
  constexpr int OKM = 0, OKR = TM::BYTES, KB = OKR + (DR > 0 ? TR::BYTES : 0);  // one K stage
  constexpr int DB = HP * TD::BYTES;                         // one dS^T stage
  constexpr int OD = 2 * KB;                                 // K stages 0, 1, then dS^T stages 0..2
  constexpr int STAGES = OD + 3 * DB;
  constexpr int SMEM = STAGES > kDenseKeyTile * (DQK + DM) * 2 ? STAGES : kDenseKeyTile * (DQK + DM) * 2;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  if ((int)blockIdx.x < a.n_split) {  // a split key tile of the KV-major kernel (DV = DM)
    combine_split_tile<DM, DR, DM>(a, blockIdx.x, smem);
    return;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = w / WPH, fh = w & 1, rs = (w % WPH) >> 1;
  const int l16 = lane & 15, g = lane >> 4, jj = l16 >> 2, qq = l16 & 3;

  // query tiles longest first (the table's order), the KV heads of one query tile together:
  // longest-first over the whole grid, and with n2 = 8 each XCD (workgroup i runs on XCD
  // i mod 8) keeps one KV head's K tiles in its L2
  const int wg = (int)blockIdx.x - a.n_split;
  const int qi = wg / a.n2, kvh = wg - qi * a.n2;
  const int b = a.tiles[2 * qi], qt = a.tiles[2 * qi + 1];
  const int64_t qs = a.cu_q[b], ks = a.cu_kv[b];
  const int S1 = (int)(a.cu_q[b + 1] - qs), S2 = (int)(a.cu_kv[b + 1] - ks);
  // the query tile's key tiles [klo, klo + nkt_run), whose dS blocks start at block blk0
  const int gq = a.qt_base[b] + qt;
  const int klo = a.qt_kr[2 * gq];
  const int nkt_run = a.qt_kr[2 * gq + 1] - klo;
  const int nvalid = min(kT, S1 - qt * kT);
  const int64_t blk0 = a.qt_blk[gq];
  const uint32_t smem_lds = lds_addr(smem);

  KeyPartLanes<WM> pm;
  KeyPartLanes<WR> pr;
  KeyPartLanes<8> pd;
  pm.init(w, lane);
  if constexpr (DR > 0) pr.init(w, lane);
  pd.init(w, lane);
  // dQ^T = K^T dS^T: the K^T fragments are the A operands, so a C tile holds features by lane
  // group and query rows by lane.  This wave's NF feature tiles are permuted: in tile f, lane
  // group g holds features F0(f) + 8 g + 4 (f % 2) + (0..3), F0(f) = fh DQK/2 + 32 (f / 2), so
  // the tile pair (2j, 2j + 1) gives each lane 8 consecutive features of one row (one 16-byte
  // store, straight from registers).  The K column reads follow: piece qq of tile f is chunk
  // group F0(f) / 32 of the K tile (RowTile::colK) plus 8 (f % 2) bytes.  Resolved now so that
  // the step loop indexes only by compile-time f: [f][ks2][first / second read].
  uint32_t kcol[NF][2][2];
  static_for<NF>([&](auto fc) {
    constexpr int f = decltype(fc)::value;
    constexpr int F0a = 32 * (f / 2), F0b = DQK / 2 + 32 * (f / 2);  // fh = 0 / 1
    auto tile = [&](auto F0c) -> int {
      constexpr int F0 = decltype(F0c)::value;
      if constexpr (F0 < DM) return OKM + TM::colK(lane, F0 / 32) + 8 * (f % 2);
      else return OKR + TR::colK(lane, (F0 - DM) / 32) + 8 * (f % 2);
    };
    constexpr int rba = F0a < DM ? TM::RB : TR::RB, rbb = F0b < DM ? TM::RB : TR::RB;
    const int base = fh ? tile(std::integral_constant<int, F0b>{}) : tile(std::integral_constant<int, F0a>{});
    const int rb = fh ? rbb : rba;
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      kcol[f][ks2][0] = base + ks2 * 32 * rb;
      kcol[f][ks2][1] = base + ks2 * 32 * rb + 16 * rb;
    }
  });
  // dS^T column reads of this wave's row tiles rt: rows (columns of the block) 16(RT rs + rt)..
  int dsA[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) dsA[rt] = TD::off(4 * g + jj, 2 * (RT * rs + rt) + (qq >> 1)) + 8 * (qq & 1);

  const uint32_t rs_m = (uint32_t)a.n2 * DM * 2, rs_r = (uint32_t)a.n2 * DR * 2;

  for (int hp0 = 0; hp0 < a.G; hp0 += HP) {
    const int h0 = kvh * a.G + hp0;  // first query head of this pass

    // transfers: wave w fills 1 KB blocks w + 8k of each part
    auto issue_part = [&](auto wtag, auto nttag, const auto& pl, const char* gtile, uint32_t rs, uint32_t lds_part,
                          int nrows) {
      constexpr int W = decltype(wtag)::value;
      constexpr bool NTL = decltype(nttag)::value;
      constexpr int RPI = RowTile<W>::RPI;
      static_for<W / 8>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const int r = min(pl.row0 + 8 * RPI * k, nrows - 1);
        const char* src = gtile + __umul24((uint32_t)r, rs) + pl.gchunk;
        if constexpr (NTL) dma16_nt<8192 * k>(src, lds_part + w * 1024);
        else dma16<8192 * k>(src, lds_part + w * 1024);
      });
    };
    // the K tile (both parts) of the range's key tile kt (key tile klo + kt), into K stage kt & 1
    auto issue_k = [&](int kt) {
      const int nk = min(kT, S2 - (klo + kt) * kT);
      const int64_t kr0 = (ks + (int64_t)(klo + kt) * kT) * a.n2 + kvh;
      const uint32_t stage = smem_lds + (kt & 1) * KB;
      issue_part(std::integral_constant<int, WM>{}, std::false_type{}, pm,
                 reinterpret_cast<const char*>(a.k + kr0 * DM), rs_m, stage + OKM, nk);
      if constexpr (DR > 0)
        issue_part(std::integral_constant<int, WR>{}, std::false_type{}, pr,
                   reinterpret_cast<const char*>(a.k_rope + kr0 * DR), rs_r, stage + OKR, nk);
    };
    // the HP dS^T blocks of key tile kt, into dS^T stage kt mod 3: HP transfers per wave
    auto issue_d = [&](int kt) {
      const uint32_t stage = smem_lds + OD + (kt % 3) * DB;
      const int64_t blk = blk0 + kt;
      const char* dblk = reinterpret_cast<const char*>(a.ds + (blk * a.n1 + h0) * (kT * kT));
      static_for<HP>([&](auto hc) {
        constexpr int hx = decltype(hc)::value;
        issue_part(std::integral_constant<int, 8>{}, std::true_type{}, pd, dblk + hx * (kT * kT * 2), kT * 2,
                   stage + hx * TD::BYTES, kT);
      });
    };

    f32x4 acc[RT][NF];  // C tile (f, rt) of dQ^T
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[rt][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    wait_vmcnt<0>();
    __syncthreads();  // every wave is done with the previous pass's stages
    // issue order K0 D0 D1, then per step kt: K(kt+1) D(kt+2).  At the top of step kt the
    // transfers issued after those of tile kt are at most D(kt+1), HP per wave (in-order
    // completion of vector loads).
    if (nkt_run > 0) {
      issue_k(0);
      issue_d(0);
    }
    if (nkt_run > 1) issue_d(1);
    for (int kt = 0; kt < nkt_run; ++kt) {
      if (kt + 1 < nkt_run) wait_vmcnt<HP>();
      else wait_vmcnt<0>();
      barrier_no_vm_wait();  // tile kt is in LDS; stages of tile kt - 1 are free
      const uint32_t stage = smem_lds + (kt & 1) * KB, dstage = smem_lds + OD + (kt % 3) * DB;
      if (kt + 1 < nkt_run) issue_k(kt + 1);
      if (kt + 2 < nkt_run) issue_d(kt + 2);
      // items i = (ks2, rt): one dS^T column fragment each, PD items ahead of its MFMAs; per
      // ks2, NF column fragments of K (those of ks2 = 1 read during ks2 = 0)
      auto kfrag = [&](int f, int ks2) -> bf16x8 {
        return join8(lds_tr16_at(stage + kcol[f][ks2][0]), lds_tr16_at(stage + kcol[f][ks2][1]));
      };
      auto dfrag = [&](int i) -> bf16x8 {
        const int ks2 = i / RT, rt = i % RT;
        const uint32_t o = dstage + hh * TD::BYTES + dsA[rt] + ks2 * 32 * TD::RB;
        return join8(lds_tr16_at(o), lds_tr16_at(o + 16 * TD::RB));
      };
      constexpr int NI = 2 * RT, PD = NI < 3 ? NI : 3;
      bf16x8 kb0[NF], kb1[NF], dring[PD];
#pragma unroll
      for (int f = 0; f < NF; ++f) kb0[f] = kfrag(f, 0);
#pragma unroll
      for (int i = 0; i < PD; ++i) dring[i] = dfrag(i);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const bf16x8 da = dring[i % PD];
        if (i + PD < NI) dring[i % PD] = dfrag(i + PD);
        if (i == 0) {
#pragma unroll
          for (int f = 0; f < NF; ++f) kb1[f] = kfrag(f, 1);
        }
        const int rt = i % RT;
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[rt][f] = mfma_16x16x32(i < RT ? kb0[f] : kb1[f], da, acc[rt][f]);
      }
      // schedule: the first reads, then per item its MFMAs followed by the reads of the item
      // PD ahead (and after item 0 the K fragments of ks2 = 1)
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * NF + 2 * PD, 0);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, NF, 0);
        if (i + PD < NI) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        if (i == 0) __builtin_amdgcn_sched_group_barrier(0x100, 2 * NF, 0);
      }
    }

    // ---- epilogue: lane l16 of row tile rt holds row 16 (RT rs + rt) + l16 of head hh and,
    // per tile pair j, features F0(2j) + 8 g .. + 7: one 16-byte store each
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = 16 * (RT * rs + rt) + l16;
      if (r < nvalid) {
        const int64_t qr = (qs + (int64_t)qt * kT + r) * a.n1 + h0 + hh;
#pragma unroll
        for (int jp = 0; jp < NF / 2; ++jp) {
          f32x4 lo = acc[rt][2 * jp], hi = acc[rt][2 * jp + 1];
#pragma unroll
          for (int i = 0; i < 4; ++i) { lo[i] *= a.scale; hi[i] *= a.scale; }
          const int d = fh * (DQK / 2) + 32 * jp + 8 * g;
          uint16_t* dst = d < DM ? a.dq + qr * DM + d : a.dq_rope + qr * DR + (d - DM);
          *reinterpret_cast<bf16x8*>(dst) = pack8(lo, hi);
        }
      }
    }
  }
}

template <int DM, int DR>
hipError_t launch_hp(const DqArgs& k, int G, dim3 grid, hipStream_t s) {
  if (G % 4 == 0) hipLaunchKernelGGL((dense_dq_ds_kernel<DM, DR, 4>), grid, dim3(512), 0, s, k);
  else if (G % 2 == 0) hipLaunchKernelGGL((dense_dq_ds_kernel<DM, DR, 2>), grid, dim3(512), 0, s, k);
  else hipLaunchKernelGGL((dense_dq_ds_kernel<DM, DR, 1>), grid, dim3(512), 0, s, k);
  return hipGetLastError();
}

}  // namespace

static hipError_t launch_dq_any(const DenseArgs& a, bool with_dq, hipStream_t s) {
  const int n_q = with_dq ? a.n_q_tiles : 0;
  if (n_q == 0 && a.n_kv_split == 0) return hipSuccess;
  DqArgs k{};
  k.k = (const uint16_t*)a.k; k.k_rope = (const uint16_t*)a.k_rope;
  k.ds = (const uint16_t*)a.ds;
  k.dq = (uint16_t*)a.dq; k.dq_rope = (uint16_t*)a.dq_rope;
  k.cu_q = a.cu_q; k.cu_kv = a.cu_kv; k.qt_base = a.qt_base; k.qt_blk = a.qt_blk; k.qt_kr = a.qt_kr;
  k.tiles = a.q_tiles;
  k.n1 = a.n1; k.n2 = a.n2; k.G = a.G;
  k.scale = a.scale;
  k.n_q_tiles = n_q;
  k.split = a.kv_split; k.part = (const float*)a.kv_part;
  k.dk = (uint16_t*)a.dk; k.dk_rope = (uint16_t*)a.dk_rope; k.dv = (uint16_t*)a.dv;
  k.n_split = a.n_kv_split;
  const dim3 grid(a.n_kv_split + n_q * a.n2);
  if (a.d_main == 128 && a.d_rope == 64) return launch_hp<128, 64>(k, a.G, grid, s);
  if (a.d_main == 128 && a.d_rope == 0) return launch_hp<128, 0>(k, a.G, grid, s);
  if (a.d_main == 64 && a.d_rope == 0) return launch_hp<64, 0>(k, a.G, grid, s);
  return hipErrorInvalidValue;
}

// dQ from the stored dS, together with the split key tiles of the KV-major kernel
hipError_t launch_dense_dq_from_ds(const DenseArgs& a, hipStream_t s) { return launch_dq_any(a, true, s); }

// the split key tiles alone (dQ recomputed elsewhere)
hipError_t launch_dense_kv_combine(const DenseArgs& a, hipStream_t s) { return launch_dq_any(a, false, s); }

}  // namespace ab
