// Selected (NSA) backward, KV-major: dK and dV of one selected block in registers, and the
// block's share of dQ for every (token, slot) that selected it (bf16 or fp16 MFMA, fp32
// accumulation; P and dS are rounded to the element type for their products).
//
// Page "NsaSelectedAttentionGrad", formula section: each query token gathers
// selectedBlockCount blocks of selectedBlockSize key / value rows through topkIndices
// (selectedKey = Gather(key, topkIndices[i]), likewise for value), then the backward of
// attention over the gathered rows: dV = P^T dY, dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d).
// The gradient of a gather is a scatter-add onto the gathered rows; here it is formed
// per block instead: the inverted index lists, for each (KV head, block), the (token,
// slot) entries that selected it in ascending order, and one workgroup owns the block.
//
// One workgroup (4 waves) owns a block of up to KB = 64 or 128 key rows of one KV head.
// Query rows stream past in steps of 64 rows = floor(64 / G) listed entries x the G query
// heads of the KV head (rows past that product are padding and contribute nothing).
// KB = 64: the waves form a 2 x 2 grid as in the dense KV-major kernel, wave w owning
// keys 32(w&1) .. +31 and rows 32(w>>1) .. +31 of every step; KB = 128: wave w owns keys
// 32w .. +31 and takes both 32-row halves of the step in turn.  K and V of a wave's keys
// stay resident in registers.  Per step:
//   S = Q K^T, dP = dY V^T, P = exp2(S*scale*log2e - lse2), dS = P (dP - drow)
//   dV += P^T dY, dK += dS^T Q                       (registers, summed over all entries)
//   dS^T -> LDS, then dQ_part^T = K^T dS^T over the block's keys (K staged in LDS once):
//   every wave owns half of the feature columns for 32 rows, and each lane stores 8
//   consecutive features of one row (bf16, 16 bytes) into the share of its (token, slot,
//   KV head): G x DQK values at dq_part[t - t0, slot, kvh], whose index is (list entry
//   t cnt + slot - t0 cnt) n2 + kvh.  Inside a share the 16-byte chunks are laid out so that
//   one store instruction writes contiguous lines (share_chunk below); the reduction puts
//   them back in (head, feature) order.
// dq_reduce_kernel then sums the slots of each (token, KV head) in slot order.  Every
// output row has one writer; no floating-point atomics: deterministic.
//
// Windows: the query tokens are cut into windows [t0, t1) so that the dQ shares of one
// window fit a bounded buffer; each window is one launch of this kernel and one of the
// reduction.  Since a list is ascending in t, a window's entries are a contiguous part
// of it (wofs).  Between windows the fp32 dK / dV accumulators of every block are kept in
// kvacc (the first window starts from zero, the last one writes the bf16 outputs).
//
// Row staging: each transfer instruction reads whole rows straight into one of two swizzled
// LDS stages (global_load_lds), the rows of step st + 2 as soon as step st no longer needs
// its stage; the list entries go the same way four steps ahead, and lanes exchange row
// tokens with __shfl.
#include "common.hpp"
#include "kernels.hpp"
#include "share_layout.hpp"

namespace ab {

namespace {

constexpr int kRows = 64;  // query rows per step
typedef __attribute__((address_space(3))) void lds_void;

struct SkvArgs {
  const uint16_t* q; const uint16_t* k; const uint16_t* v; const uint16_t* dy;
  const float* lse2; const float* ndrow;
  uint16_t* dk; uint16_t* dv;
  uint16_t* dq_part;          // [window tokens, cnt, n2, G, DQK] in the element type
  int trash_row;              // first of G share rows after those of the window: rows without an
                              // entry store there (never read), so every step issues the same stores
  const int64_t* cu_kv;
  const int32_t* blkoff;      // [B+1] blocks before each sequence
  const int32_t* offsets;     // inverted index: [n2 * nblk_total + 1]
  const int32_t* list;        // entries t * cnt + slot, ascending per (KV head, block)
  const int32_t* sched;       // [n2 * nblk_total] work order: keys by length class, then key
  const int32_t* wofs;        // [n2 * nblk_total, nwin + 1] list position where each window starts
  float* kvacc;               // fp32 dK / dV of every key between windows, KB (DQK + DV) per key
  int batch, n1, n2, G, bs, cnt, nblk_total;
  int nwin, win;              // windows of query tokens; this launch takes window `win`
  int e_lo;                   // first list entry (t cnt + slot) of the window: share row 0
  float scale, scale_log2e;
};

__device__ __forceinline__ void barrier_no_vm_wait() {
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

// 4 bytes per lane from global memory into LDS at M0 = lds, + 4 * lane
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               ::"v"(src), "s"(lds) : "memory", "m0");
}

// s_waitcnt operand for vmcnt(n) lgkmcnt(0), export count not waited for
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70; }
static_assert(wait_vm_lgkm0(63) == 0xc07f && wait_vm_lgkm0(0) == 0x0070, "s_waitcnt encoding");

template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for_i(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_i<N, F, I + 1>(static_cast<F&&>(f));
  }
}

__device__ __forceinline__ uint32_t lds_addr(const void* lds) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds);
}

// Staging of one part (RowTile of W chunks) by one wave: transfer kk of wave w writes rows
// (w + 4 kk) RPI + lane / W, slot lane % W, i.e. the lane reads chunk (lane % W) ^ swz(row),
// the same chunk for every kk.  Operand reads use RowTile::rowA / colB / colK.
template <int W>
struct PartLanes {
  using T = RowTile<W>;
  int row0;
  uint32_t gchunk;
  __device__ __forceinline__ void init(int w, int lane) {
    row0 = w * T::RPI + lane / W;
    gchunk = 16u * (uint32_t)((lane % W) ^ T::swz(row0));
  }
};

template <typename T, int DM, int DR, int DV, int KB>
__global__ __launch_bounds__(256, 1) void sel_kv_kernel(SkvArgs a) {
  using V8 = typename Mma<T>::v8;
  static_assert(KB == 64 || KB == 128, "64 or 128 keys per workgroup");
  constexpr int NRH = KB / 64;  // 32-row halves of a step taken by each wave
  constexpr int DQK = DM + DR;
  constexpr int KS = DQK / 32, VS = DV / 32, NQ = DQK / 16, NV = DV / 16;
  constexpr int KSM = DM / 32, NQM = DM / 16;
  constexpr int WM = DM / 8, WR = DR > 0 ? DR / 8 : 8, WY = DV / 8;
  constexpr int NFH = NQ / 2;  // dQ-part feature tiles per wave (half of the features)
  using TM = RowTile<WM>;
  using TR = RowTile<WR>;
  using TY = RowTile<WY>;
  using TD = RowTile<8>;       // dS^T tile: 64 keys x 64 rows
  constexpr int OQM = 0, OQR = TM::BYTES, OY = OQR + (DR > 0 ? TR::BYTES : 0);
  // stage: QM, QR, Y, then 4 x 256 bytes of row statistics (lse2 from wave 0, ndrow from wave
  // 1; waves 2 and 3 load the same rows into the other two slots, which nothing reads)
  constexpr int OL = OY + TY::BYTES, ORW = OL + 256, SB = OL + 1024;
  constexpr int OKM = 2 * SB, OKR = OKM + NRH * TM::BYTES;            // K tile, KB rows (dQ product)
  constexpr int ODS = OKR + (DR > 0 ? NRH * TR::BYTES : 0);           // dS^T tile, KB key rows
  constexpr int OENT = ODS + NRH * TD::BYTES;                          // per wave: 4 steps of list entries
  constexpr int NACC = 2 * (NQ + NV);
  constexpr int EPI = (NRH == 1 ? 2 * NACC * 1024 : 0) + KB * (DQK + DV) * 2;
  constexpr int MAIN = OENT + 4 * 1024;
  constexpr int SMEM = MAIN > EPI ? MAIN : EPI;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  static_assert(SB % 256 == 0 && OQR % 256 == 0 && OY % 256 == 0 && OKM % 256 == 0 && OKR % 256 == 0,
                "part bases keep bits 0-7 clear (XOR operand addressing)");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = NRH == 1 ? (w & 1) : w;      // key group: keys 32 kh .. +31
  const int rh0 = NRH == 1 ? (w >> 1) : 0;    // first 32-row half of the step
  const int qh = w >> 1;                      // dQ product: rows 32 qh .. +31
  const int l16 = lane & 15, g = lane >> 4;

  // ---- work unit: (KV head, block) and its list of entries -------------------------
  const int u = a.sched[blockIdx.x];
  const int kvh = u / a.nblk_total;
  const int rem = u - kvh * a.nblk_total;
  const int b = seq_of32(a.blkoff, a.batch, rem);
  const int64_t k0 = a.cu_kv[b] + (int64_t)(rem - a.blkoff[b]) * a.bs;
  const int nk = a.bs;
  // the entries of this window: a contiguous part of the (ascending) list
  const int e_begin = a.nwin > 1 ? a.wofs[(int64_t)u * (a.nwin + 1) + a.win] : a.offsets[u];
  const int e_end = a.nwin > 1 ? a.wofs[(int64_t)u * (a.nwin + 1) + a.win + 1] : a.offsets[u + 1];
  const bool first_win = a.win == 0, last_win = a.win == a.nwin - 1;
  // a window between the first and the last with no entry leaves the accumulators as they are
  if (e_begin == e_end && !first_win && !last_win) return;  // whole workgroup
  const int G = a.G, TPS = kRows / G;  // entries per step
  const int nsteps = (e_end - e_begin + TPS - 1) / TPS;
  const int hh_row = lane % G;  // head (within the group) of step row `lane`

  // ---- resident keys: K and V as MFMA B operands; K also staged in LDS for dQ --------
  V8 Kf[2][KS], Vf[2][VS];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = 32 * kh + 16 * t + l16;
    const bool valid = key < nk;
    const int64_t kr = (k0 + key) * a.n2 + kvh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (valid) x = ldg16(a.k + kr * DQK + 32 * s + 8 * g);
      Kf[t][s] = as_v8<T>(x);
    }
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (valid) x = ldg16(a.v + kr * DV + 32 * s + 8 * g);
      Vf[t][s] = as_v8<T>(x);
    }
  }

  PartLanes<WM> pm;
  PartLanes<WR> pr;
  PartLanes<WY> py;
  pm.init(w, lane);
  if constexpr (DR > 0) pr.init(w, lane);
  py.init(w, lane);
  const uint32_t smem_lds = lds_addr(smem);

  // K tile in LDS (RowTile layout, KB key rows; keys past the block repeat its last key).
  // The dQ product reads it by columns, every lane the same 8-byte half of its chunk; two
  // rows whose swizzles differ by 2 (bit 1 of swz, see khalf) would read the same chunks,
  // so on the rows with that bit set the two halves of every chunk are swapped.
  auto khalf = [](auto tile, int r) -> int { return (decltype(tile)::swz(r) >> 1) & 1; };
  auto half_swap = [](uint4 x, int sw) -> uint4 { return sw ? make_uint4(x.z, x.w, x.x, x.y) : x; };
  {
    PartLanes<WM> km;
    km.init(w, lane);
#pragma unroll
    for (int hk = 0; hk < NRH; ++hk)
#pragma unroll
      for (int kk = 0; kk < WM / 4; ++kk) {
        const int rl = 64 * hk + km.row0 + 4 * TM::RPI * kk;  // row of the tile
        const int r = min(rl, nk - 1);
        const uint4 x = ldg16(reinterpret_cast<const char*>(a.k + ((k0 + r) * a.n2 + kvh) * DQK) + km.gchunk);
        lds_st16_at(smem_lds + OKM + hk * TM::BYTES + (w + 4 * kk) * 1024 + 16 * lane, half_swap(x, khalf(TM{}, rl)));
      }
    if constexpr (DR > 0) {
      PartLanes<WR> kr_;
      kr_.init(w, lane);
#pragma unroll
      for (int hk = 0; hk < NRH; ++hk)
#pragma unroll
        for (int kk = 0; kk < WR / 4; ++kk) {
          const int rl = 64 * hk + kr_.row0 + 4 * TR::RPI * kk;
          const int r = min(rl, nk - 1);
          const uint4 x =
              ldg16(reinterpret_cast<const char*>(a.k + ((k0 + r) * a.n2 + kvh) * DQK + DM) + kr_.gchunk);
          lds_st16_at(smem_lds + OKR + hk * TR::BYTES + (w + 4 * kk) * 1024 + 16 * lane, half_swap(x, khalf(TR{}, rl)));
        }
    }
  }
  // dQ product split: wave w owns feature half fh = w & 1 and rows 32 rh .. +31 of the
  // step.  Its NFH feature tiles are permuted: in C tile f, lane group g holds features
  // F0(f) + 8 g + 4 (f % 2) + (0..3) with F0(f) = fh DQK/2 + 32 (f / 2), so the tile pair
  // (2j, 2j+1) gives each lane 8 consecutive features (one 16-byte store) and the four
  // lane groups of a row cover 64 consecutive bytes.  The K^T column reads follow the
  // permutation: 4-feature piece qq of tile f starts at feature F0(f) + 8 qq + 4 (f % 2),
  // i.e. chunk group F0(f) / 32 of the K tile (RowTile::colK) plus 8 (f % 2) bytes, that
  // half swapped on the lane's row if khalf says so (the row parity a lane reads is the
  // same for every tile, k-step and +16 rows).
  const int fh = w & 1;
  const uint32_t kcm = smem_lds + OKM + TM::colK(lane, 0);
  const uint32_t kcr = smem_lds + OKR + TR::colK(lane, 0);
  const uint32_t khm = 8u * khalf(TM{}, 4 * g + (l16 >> 2)), khr = 8u * khalf(TR{}, 4 * g + (l16 >> 2));
  int dscol[2], rmod[2];  // column reads of the dS^T tile; head of dQ-product rows 32 qh + 16 rr + l16
  int schunk[2];           // share chunk of piece 0 for those rows (share_chunk)
  const int SR = share_rows(G);
  {
    const int jj = l16 >> 2, qq = l16 & 3;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      dscol[rr] = ODS + TD::off(4 * g + jj, 2 * (2 * qh + rr) + (qq >> 1)) + 8 * (qq & 1);
      rmod[rr] = (32 * qh + 16 * rr + l16) % G;
      schunk[rr] = share_chunk<DQK>(rmod[rr], 4 * fh * (NFH / 2) + g, SR);
    }
  }

  // dK / dV accumulators of this window (the sums of earlier windows are added at the end)
  f32x4 dK[2][NQ], dV[2][NV];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) dK[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NV; ++n) dV[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- list entries: row `lane` of step st is entry e_begin + st * TPS + lane / G ------
  // (-1 for padding rows and rows past the list)
  auto row_has = [&](int st) -> bool {
    const int slot = lane / G;  // entry slot of row `lane`; slots >= TPS are padding rows
    return slot < TPS && e_begin + st * TPS + slot < e_end;
  };
  auto entry_of = [&](int st) -> int { return row_has(st) ? a.list[e_begin + st * TPS + lane / G] : -1; };
  const int first_entry = e_begin < e_end ? a.list[e_begin] : 0;  // stands in for missing rows
  // rows of step st that have an entry: a prefix of the step (entry-major rows)
  auto rows_valid = [&](int st) -> int { return min(TPS, e_end - e_begin - st * TPS) * G; };

  // ---- staging ------------------------------------------------------------------------
  // Every transfer goes from global memory straight into LDS (global_load_lds), so that no
  // registers hold a stage and the rows of step st + 2 are requested as soon as the stage
  // of step st is free (after the waves' S / dP products of step st), about 1.25 steps
  // before they are used.  The list entries travel the same way, 4 steps ahead, into a
  // 4-slot ring of this wave (lane = row of the step).  All transfers and stores of a step
  // are issued whatever the step (rows past the list read the first entry's rows, entries
  // past it the first entry), so the number of vector-memory operations each wave issues
  // per step is fixed and the wait before a step counts exactly what may stay in flight.
  const uint32_t ring = smem_lds + OENT + 1024 * w;
  // Rows this lane transfers for the stage being prepared, as row indices t n1 + h of the
  // [T1, n1, D] tensors (below 2^28: T1 is at most 2M and N1 at most 128): the row tokens
  // are exchanged between lanes (LDS permutes, issued together).
  int rim[WM / 4], rir[WR / 4], riy[WY / 4], rist = 0;
  auto prep_rows = [&](int ent) {  // ent: this lane's entry for its row (row = lane) of the step
    const int tok_lane = (ent >= 0 ? ent : first_entry) / a.cnt;
    int tm[WM / 4], tr[WR / 4], ty[WY / 4];
#pragma unroll
    for (int kk = 0; kk < WM / 4; ++kk) tm[kk] = __shfl(tok_lane, pm.row0 + 4 * TM::RPI * kk);
    if constexpr (DR > 0) {
#pragma unroll
      for (int kk = 0; kk < WR / 4; ++kk) tr[kk] = __shfl(tok_lane, pr.row0 + 4 * TR::RPI * kk);
    }
#pragma unroll
    for (int kk = 0; kk < WY / 4; ++kk) ty[kk] = __shfl(tok_lane, py.row0 + 4 * TY::RPI * kk);
    const int h0 = kvh * G;
#pragma unroll
    for (int kk = 0; kk < WM / 4; ++kk) rim[kk] = tm[kk] * a.n1 + h0 + (pm.row0 + 4 * TM::RPI * kk) % G;
    if constexpr (DR > 0) {
#pragma unroll
      for (int kk = 0; kk < WR / 4; ++kk) rir[kk] = tr[kk] * a.n1 + h0 + (pr.row0 + 4 * TR::RPI * kk) % G;
    }
#pragma unroll
    for (int kk = 0; kk < WY / 4; ++kk) riy[kk] = ty[kk] * a.n1 + h0 + (py.row0 + 4 * TY::RPI * kk) % G;
    rist = tok_lane * a.n1 + h0 + hh_row;
  };
  // the rows found by prep_rows into the stage at `stage`: this wave's 1 KB blocks of each
  // part, and the row statistic (lse2 for even waves, ndrow for odd) of the 64 rows
  auto issue_stage = [&](uint32_t stage) {
    static_for_i<WM / 4>([&](auto kc) {
      constexpr int kk = decltype(kc)::value;
      dma16<4096 * kk>(reinterpret_cast<const char*>(a.q + (int64_t)rim[kk] * DQK) + pm.gchunk, stage + OQM + 1024 * w);
    });
    if constexpr (DR > 0) {
      static_for_i<WR / 4>([&](auto kc) {
        constexpr int kk = decltype(kc)::value;
        dma16<4096 * kk>(reinterpret_cast<const char*>(a.q + (int64_t)rir[kk] * DQK + DM) + pr.gchunk,
                         stage + OQR + 1024 * w);
      });
    }
    static_for_i<WY / 4>([&](auto kc) {
      constexpr int kk = decltype(kc)::value;
      dma16<4096 * kk>(reinterpret_cast<const char*>(a.dy + (int64_t)riy[kk] * DV) + py.gchunk, stage + OY + 1024 * w);
    });
    dma4(((w & 1) ? a.ndrow : a.lse2) + rist, stage + OL + 256 * w);
  };
  // the list entries of step st into ring slot st % 4 (entries past the list read the first)
  auto issue_entries = [&](int st) {
    dma4(a.list + (row_has(st) ? e_begin + st * TPS + lane / G : e_begin), ring + 256 * (st & 3));
  };
  auto ring_entry = [&](int st) -> int {
    const int e = __builtin_bit_cast(int, lds_f32_at(ring + 256 * (st & 3) + 4 * lane));
    return row_has(st) ? e : -1;
  };
  // vector-memory operations per step: the stage's transfers, the entries, the dQ-share stores
  constexpr int NSO = WM / 4 + (DR > 0 ? WR / 4 : 0) + WY / 4 + 1, NST = NFH;

  // ---- one step ------------------------------------------------------------------------
  // rows 32 (rh0 + hi) .. +31 of the step staged at `stage`, whose first nvr rows have an
  // entry: S, dP, P, dS, dS^T -> LDS, dV += P^T dY, dK += dS^T Q
  auto half_step = [&](uint32_t stage, auto hic, int nvr) {
    constexpr int hi = decltype(hic)::value;
    const int rh = rh0 + hi;
    // lane bases of this wave's first row half (256-byte aligned part bases; see RowTile)
    const uint32_t vm = stage + OQM + rh0 * 32 * TM::RB, vr = stage + OQR + rh0 * 32 * TR::RB;
    const uint32_t vy = stage + OY + rh0 * 32 * TY::RB;
    const uint32_t statb = opaque(stage + OL + 4 * (32 * rh + 4 * g));  // lse2; ndrow at + 256
    f32x4 lse[2], ndr[2];  // ndrow = -drow: the dP accumulators start there and end at dP - drow
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      lse[rt] = lds_f32x4_at(statb + 64 * rt);
      ndr[rt] = lds_f32x4_at(statb + 256 + 64 * rt);
    }
    if (nvr < kRows) {  // rows without an entry (their rows are the first entry's): P = 0, no drow
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool pad = 32 * rh + 16 * rt + 4 * g + i >= nvr;
          lse[rt][i] = pad ? INFINITY : lse[rt][i];
          ndr[rt][i] = pad ? 0.f : ndr[rt][i];
        }
    }
    constexpr int NS = KS + VS, PA = KB == 128 ? 2 : 3;  // A-fragment reads in flight
    const uint32_t am = vm + TM::rowA(lane, 0), ar = vr + TR::rowA(lane, 0), ay = vy + TY::rowA(lane, 0);
    auto afrag = [&](int s, int rt) -> V8 {
      if (s < KSM) return as_v8<T>(lds_b128_at((am ^ (64u * s)) + (32 * hi + 16 * rt) * TM::RB));
      if (s < KS) return as_v8<T>(lds_b128_at((ar ^ (64u * (s - KSM))) + (32 * hi + 16 * rt) * TR::RB));
      return as_v8<T>(lds_b128_at((ay ^ (64u * (s - KS))) + (32 * hi + 16 * rt) * TY::RB));
    };
    V8 aring[PA][2];
#pragma unroll
    for (int i = 0; i < PA; ++i) { aring[i][0] = afrag(i, 0); aring[i][1] = afrag(i, 1); }
    f32x4 S[2][2], D[2][2];  // [key tile][row tile]
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const V8 a0 = aring[s % PA][0], a1 = aring[s % PA][1];
      if (s + PA < NS) { aring[s % PA][0] = afrag(s + PA, 0); aring[s % PA][1] = afrag(s + PA, 1); }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (s < KS) {
          S[t][0] = Mma<T>::run(a0, Kf[t][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : S[t][0]);
          S[t][1] = Mma<T>::run(a1, Kf[t][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : S[t][1]);
        } else {
          D[t][0] = Mma<T>::run(a0, Vf[t][s - KS], s == KS ? ndr[0] : D[t][0]);
          D[t][1] = Mma<T>::run(a1, Vf[t][s - KS], s == KS ? ndr[1] : D[t][1]);
        }
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PA, 0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      if (s + PA < NS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    // P (keys past the block -> 0; a wave-uniform test first, blocks are mostly full), then
    // dS in place
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t][rt][i] = __builtin_amdgcn_exp2f(S[t][rt][i] * a.scale_log2e - lse[rt][i]);
    if (32 * kh + 32 > nk) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bool kvalid = 32 * kh + 16 * t + l16 < nk;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) S[t][rt][i] = kvalid ? S[t][rt][i] : 0.f;
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) D[t][rt][i] = S[t][rt][i] * D[t][rt][i];
    V8 pa[2], da[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      pa[t] = pack8t<T>(S[t][0], S[t][1]);
      da[t] = pack8t<T>(D[t][0], D[t][1]);
      // dS^T tile: key 32kh + 16t + l16, rows 32rh + 4g + (0..3) and + 16 (8-byte writes)
      const i16x8 d8 = __builtin_bit_cast(i16x8, da[t]);
      const int key = 32 * kh + 16 * t + l16;
      const int r0 = 32 * rh + 4 * g;
      const uint32_t o0 = smem_lds + ODS + TD::off(key, r0 >> 3) + 2 * (r0 & 7);
      const uint32_t o1 = smem_lds + ODS + TD::off(key, (r0 + 16) >> 3) + 2 * ((r0 + 16) & 7);
      *reinterpret_cast<__attribute__((address_space(3))) i16x4*>((uintptr_t)o0) = i16x4{d8[0], d8[1], d8[2], d8[3]};
      *reinterpret_cast<__attribute__((address_space(3))) i16x4*>((uintptr_t)o1) = i16x4{d8[4], d8[5], d8[6], d8[7]};
    }
    // dV += P^T dY, dK += dS^T Q
    const uint32_t cm = vm + TM::colB(lane, 0), cr = vr + TR::colB(lane, 0), cy = vy + TY::colB(lane, 0);
    auto colfrag = [&](int j) -> V8 {
      uint32_t o;
      int rb;
      if (j < NV) { o = cy ^ (32u * j); rb = TY::RB; }
      else if (j < NV + NQM) { o = cm ^ (32u * (j - NV)); rb = TM::RB; }
      else { o = cr ^ (32u * (j - NV - NQM)); rb = TR::RB; }
      return as_v8<T>(join8(lds_tr16_at(o + 32 * hi * rb), lds_tr16_at(o + (32 * hi + 16) * rb)));
    };
    constexpr int NJ = NV + NQ, PD = KB == 128 ? 3 : 4;  // column reads in flight (128 keys: fewer registers)
    V8 ring[PD];
#pragma unroll
    for (int i = 0; i < PD; ++i) ring[i] = colfrag(i);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const V8 bj = ring[j % PD];
      if (j + PD < NJ) ring[j % PD] = colfrag(j + PD);
      if (j < NV) {
        dV[0][j] = Mma<T>::run(pa[0], bj, dV[0][j]);
        dV[1][j] = Mma<T>::run(pa[1], bj, dV[1][j]);
      } else {
        dK[0][j - NV] = Mma<T>::run(da[0], bj, dK[0][j - NV]);
        dK[1][j - NV] = Mma<T>::run(da[1], bj, dK[1][j - NV]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PD, 1);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
      if (j + PD < NJ) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }

  };

  // dQ_part^T (features x rows) = K^T dS^T over the KB keys, for the feature half FH and
  // rows 32 qh .. +31
  auto dq_prod = [&](f32x4 (&acc)[NFH][2], auto fhc) {
    constexpr int FH = decltype(fhc)::value;
#pragma unroll
    for (int f = 0; f < NFH; ++f)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) acc[f][rr] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KB / 32; ++ks) {
      V8 kt[NFH], dt[2];
      static_for_i<NFH>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        constexpr int F0 = FH * (DQK / 2) + 32 * (f / 2);
        constexpr int rb = F0 < DM ? TM::RB : TR::RB;
        const uint32_t o = (F0 < DM ? (kcm ^ (64u * (F0 / 32))) + ((8u * (f % 2)) ^ khm)
                                    : (kcr ^ (64u * ((F0 - DM) / 32))) + ((8u * (f % 2)) ^ khr)) + ks * 32 * rb;
        kt[f] = as_v8<T>(join8(lds_tr16_at(o), lds_tr16_at(o + 16 * rb)));
      });
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const uint32_t o = smem_lds + dscol[rr] + ks * 32 * TD::RB;
        dt[rr] = as_v8<T>(join8(lds_tr16_at(o), lds_tr16_at(o + 16 * TD::RB)));
      }
#pragma unroll
      for (int f = 0; f < NFH; ++f)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) acc[f][rr] = Mma<T>::run(kt[f], dt[rr], acc[f][rr]);
    }
  };
  // every row with an entry stores its share (G x DQK in the element type); C tile (f, rr):
  // the lane holds row 32 qh + 16 rr + l16 and the permuted features above (feature half fh)
  auto dq_store = [&](int ent_cur, const f32x4 (&acc)[NFH][2]) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int r = 32 * qh + 16 * rr + l16;
      const int ent = __shfl(ent_cur, r);
      // first row of the share (below 2^28: the shares of a window take at most 64 GiB)
      const int srow0 = ent >= 0 ? ((ent - a.e_lo) * a.n2 + kvh) * G : a.trash_row;
      uint16_t* dst = a.dq_part + (int64_t)srow0 * DQK + 8 * schunk[rr];
#pragma unroll
      for (int j = 0; j < NFH / 2; ++j)  // piece j: row chunk 4 (fh NFH / 2 + j) + g
        *reinterpret_cast<V8*>(dst + 8 * 4 * SR * j) = pack8t<T>(acc[2 * j][rr], acc[2 * j + 1][rr]);
    }
  };

  // step st: the S / dP products, then (the stage being free) the transfers of step st + 2
  // and the entries of step st + 4, then the dQ product and the shares
  auto step = [&](int st, int ent_cur) {
    const uint32_t stage = smem_lds + (st & 1) * SB;
    const int nvr = rows_valid(st);
    static_for_i<NRH>([&](auto hic) { half_step(stage, hic, nvr); });
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's stage reads and dS^T writes are done
    barrier_no_vm_wait();                // every wave's dS^T is in LDS; stage st is free
    issue_stage(stage);                  // rows prepared at the top of the step
    issue_entries(st + 4);
    f32x4 acc[NFH][2];
    if (fh) dq_prod(acc, std::integral_constant<int, 1>{});
    else dq_prod(acc, std::integral_constant<int, 0>{});
    dq_store(ent_cur, acc);  // after the join: one store sequence
  };

  // ---- step loop -----------------------------------------------------------------------
  // Before step st the stage of step st and the entries of step st + 2 must have arrived.
  // This wave issued after them, in order: at step 0 the stage of step 1; at step 1 the
  // operations of step 0; later the shares of step st - 2 and the operations of step st - 1
  // (see step): that many may stay in flight.
  __syncthreads();  // K tile in LDS
  if (nsteps > 0) {
    // ring slots 0, 1 from registers, 2, 3 by transfer; the stages of steps 0 and 1
    const int e0 = entry_of(0), e1 = entry_of(1);
    lds_st4_at(ring + 4 * lane, __builtin_bit_cast(float, e0));
    lds_st4_at(ring + 256 + 4 * lane, __builtin_bit_cast(float, e1));
    issue_entries(2);
    issue_entries(3);
    prep_rows(e0);
    issue_stage(smem_lds);
    prep_rows(e1);
    issue_stage(smem_lds + SB);
  }
  for (int st = 0; st < nsteps; ++st) {
    if (st >= 2) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(2 * NST + NSO + 1));
    else if (st == 1) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(NST + NSO + 1));
    else __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(NSO));
    barrier_no_vm_wait();
    const int ent_cur = ring_entry(st);
    prep_rows(ring_entry(st + 2));
    step(st, ent_cur);
  }
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));  // no transfer into LDS left in flight

  // ---- epilogue: dK, dV to bf16 through LDS (KB = 64: the two row halves summed first),
  // then 16-byte stores of whole rows.  With several windows the fp32 sums of the earlier
  // windows are added (in this fixed order: row half 0, row half 1, earlier windows), and
  // before the last window the result goes back to kvacc instead.
  // kvacc layout per key: [key group kh][t][NQ dK tiles, NV dV tiles][lane] f32x4
  f32x4* const accu = reinterpret_cast<f32x4*>(a.kvacc) + (int64_t)u * (KB / 32) * NACC * 64;
  const bool keep = !last_win;
  auto prev = [&](int i) { return first_win ? f32x4{0.f, 0.f, 0.f, 0.f} : accu[i * 64 + lane]; };
  auto keep_acc = [&](auto&& other_k, auto&& other_v) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        const int i = kh * NACC + t * (NQ + NV) + n;
        accu[i * 64 + lane] = dK[t][n] + other_k(t, n) + prev(i);
      }
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        const int i = kh * NACC + t * (NQ + NV) + NQ + n;
        accu[i * 64 + lane] = dV[t][n] + other_v(t, n) + prev(i);
      }
    }
  };
  __syncthreads();
  uint16_t* Ko = reinterpret_cast<uint16_t*>(smem + (NRH == 1 ? 2 * NACC * 1024 : 0));
  uint16_t* Vo = Ko + KB * DQK;
  auto put = [&](auto&& other_k, auto&& other_v) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        const f32x4 o = other_k(t, n);
        const f32x4 e = prev(kh * NACC + t * (NQ + NV) + n);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Ko[(32 * kh + 16 * t + 4 * g + i) * DQK + 16 * n + l16] = f2t<T>((dK[t][n][i] + o[i] + e[i]) * a.scale);
      }
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        const f32x4 o = other_v(t, n);
        const f32x4 e = prev(kh * NACC + t * (NQ + NV) + NQ + n);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Vo[(32 * kh + 16 * t + 4 * g + i) * DV + 16 * n + l16] = f2t<T>(dV[t][n][i] + o[i] + e[i]);
      }
    }
  };
  if constexpr (NRH == 1) {
    f32x4* part = reinterpret_cast<f32x4*>(smem);
    if (rh0 == 1) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int n = 0; n < NQ; ++n) part[(kh * NACC + t * (NQ + NV) + n) * 64 + lane] = dK[t][n];
#pragma unroll
        for (int n = 0; n < NV; ++n) part[(kh * NACC + t * (NQ + NV) + NQ + n) * 64 + lane] = dV[t][n];
      }
    }
    __syncthreads();
    const auto ok = [&](int t, int n) { return part[(kh * NACC + t * (NQ + NV) + n) * 64 + lane]; };
    const auto ov = [&](int t, int n) { return part[(kh * NACC + t * (NQ + NV) + NQ + n) * 64 + lane]; };
    if (rh0 == 0) {
      if (keep) keep_acc(ok, ov);
      else put(ok, ov);
    }
  } else {
    const auto zero = [](int, int) { return f32x4{0.f, 0.f, 0.f, 0.f}; };
    if (keep) keep_acc(zero, zero);
    else put(zero, zero);
  }
  if (keep) return;  // whole workgroup
  __syncthreads();
  constexpr int QCH = DQK / 8, YCH = DV / 8;
  for (int idx = tid; idx < KB * QCH; idx += 256) {
    const int r = idx / QCH, c = idx - r * QCH;
    if (r < nk) sts16(a.dk + ((k0 + r) * a.n2 + kvh) * DQK + 8 * c, *reinterpret_cast<const uint4*>(Ko + r * DQK + 8 * c));
  }
  for (int idx = tid; idx < KB * YCH; idx += 256) {
    const int r = idx / YCH, c = idx - r * YCH;
    if (r < nk) sts16(a.dv + ((k0 + r) * a.n2 + kvh) * DV + 8 * c, *reinterpret_cast<const uint4*>(Vo + r * DV + 8 * c));
  }
}

}  // namespace

// This file is compiled twice: SEL_KV_KEYS = 64 gives the kernels for blocks of up to 64
// keys (and launch_selected_kv_b64), SEL_KV_KEYS = 128 those for larger blocks plus the
// dispatching launch_selected_kv.  The two units take different code generation options.
#ifndef SEL_KV_KEYS
#error "compile with -DSEL_KV_KEYS=64 or -DSEL_KV_KEYS=128"
#endif

namespace {

template <int KB>
hipError_t launch_keys(const SelArgs& a, hipStream_t s) {
  SkvArgs k{};
  k.q = (const uint16_t*)a.q; k.k = (const uint16_t*)a.k; k.v = (const uint16_t*)a.v; k.dy = (const uint16_t*)a.dy;
  k.lse2 = a.lse2; k.ndrow = a.ndrow;
  k.dk = (uint16_t*)a.dk; k.dv = (uint16_t*)a.dv; k.dq_part = (uint16_t*)a.dq_part;
  k.trash_row = (int)(std::min<int64_t>(a.win_tokens, a.T1) * a.cnt * a.n1);
  k.cu_kv = a.cu_kv; k.blkoff = a.blkoff; k.offsets = a.offsets; k.list = a.list; k.sched = a.cursor;
  k.wofs = a.wofs; k.kvacc = a.kvacc; k.nwin = a.nwin; k.win = a.win; k.e_lo = (int)(a.t0 * a.cnt);
  k.batch = a.batch; k.n1 = a.n1; k.n2 = a.n2; k.G = a.G; k.bs = a.bs; k.cnt = a.cnt; k.nblk_total = a.nblk_total;
  k.scale = a.scale; k.scale_log2e = a.scale_log2e;
  const dim3 grid((unsigned)(a.n2 * a.nblk_total));
  if (a.is_f16) {
    if (a.d_qk == 192) hipLaunchKernelGGL((sel_kv_kernel<_Float16, 128, 64, 128, KB>), grid, dim3(256), 0, s, k);
    else hipLaunchKernelGGL((sel_kv_kernel<_Float16, 128, 0, 128, KB>), grid, dim3(256), 0, s, k);
  } else {
    if (a.d_qk == 192) hipLaunchKernelGGL((sel_kv_kernel<__bf16, 128, 64, 128, KB>), grid, dim3(256), 0, s, k);
    else hipLaunchKernelGGL((sel_kv_kernel<__bf16, 128, 0, 128, KB>), grid, dim3(256), 0, s, k);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_selected_kv_b64(const SelArgs& a, hipStream_t s);  // the SEL_KV_KEYS = 64 unit

#if SEL_KV_KEYS == 64
hipError_t launch_selected_kv_b64(const SelArgs& a, hipStream_t s) { return launch_keys<64>(a, s); }
#else
bool selected_supported(int d_qk, int d_v, int G, int bs) {
  return (d_qk == 192 || d_qk == 128) && d_v == 128 && G >= 1 && G <= 32 && bs >= 16 && bs <= 128 && bs % 16 == 0;
}

hipError_t launch_selected_kv(const SelArgs& a, hipStream_t s) {
  if (!selected_supported(a.d_qk, a.d_v, a.G, a.bs)) return hipErrorInvalidValue;
  if (a.n2 * a.nblk_total == 0) return hipSuccess;
  return a.bs > 64 ? launch_keys<128>(a, s) : launch_selected_kv_b64(a, s);
}
#endif

}  // namespace ab
