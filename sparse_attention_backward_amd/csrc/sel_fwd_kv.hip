// Selected (NSA) attention forward, KV-major with per-block partial softmax.
//
// Page "NsaSelectedAttentionGrad": the backward consumes attentionOut, softmaxMax and
// softmaxSum, the forward's outputs; for query token t and KV head n2 the G query heads
// attend to the selectedBlockCount blocks that topkIndices[t, n2] gathers:
//   s = scale Q K^T,  m = max s,  l = sum exp(s - m),  O = sum exp(s - m) V / l.
// The softmax over the gathered rows splits over the blocks: with each block's own
// m_b = max of its scores, l_b = sum exp(s - m_b) and O_b = sum exp(s - m_b) V / l_b,
//   m = max_b m_b,  l = sum_b l_b exp(m_b - m),  O = sum_b (l_b exp(m_b - m) / l) O_b.
//
// Pass 1 (sel_fwd_kv_kernel): one workgroup per (KV head, block), that block's K and V rows
// resident in LDS; the block's list of (token, slot) entries (the inverted index, ascending)
// is dealt to the four waves, each entry to one wave.  Per entry the G heads' query rows are
// gathered straight into registers as the B operand (the next entry's rows load while the
// current one computes), and the heads are the MFMA columns:
//   S^T (keys x heads) = K (A: row reads of the K tile) x Q^T,
//   m_b, P^T = exp2(S^T scale log2 e - m_b), l_b per head (column),
//   O_b^T (features x heads) = V^T (A: column reads of the V tile) x P^T / l_b.
// O_b (element type) and (m_b, l_b) (fp32, log2 domain) are stored as the entry's partial,
// row (entry - first entry of the window) N2 + KV head.  Per entry this moves the query rows
// (G D_qk elements) and a partial of G D_v elements, instead of gathering the block's
// bs (D_qk + D_v) elements of K and V for every entry.
// Pass 2 (sel_fwd_combine_kernel): one wave per (token, KV head): the cnt partials merged
// in slot order into O, softmaxMax (natural units) and softmaxSum.  Slots whose id
// is out of range have no partial (the index build skipped them and raised the flag).
//
// The same two passes give the backward's row statistic when attentionOut is not passed
// (the page lists it as optional): drow = sum_j P_j dP_j over the gathered rows, with P from
// the passed statistics and dP = dY V^T, per entry in sel_drow_kv_kernel (query and dY rows
// gathered, 10 KB per entry at G = 16, instead of the block's K and V rows) and summed over
// the slots in order by sel_drow_combine_kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

__device__ __forceinline__ float max4(f32x4 v) { return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])); }
__device__ __forceinline__ float sum4(f32x4 v) { return (v[0] + v[1]) + (v[2] + v[3]); }
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <typename T>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (T)x) | ((uint32_t)__builtin_bit_cast(uint16_t, (T)y) << 16);
}

constexpr int kDv = 128;

// LDS of a KV-major workgroup: the block's K rows (main 128 features, then the rest) and V
// rows, KB rows each (64-row RowTiles), rows past the block zero.
template <int DQK, int KB>
struct KvTiles {
  static constexpr int DR = DQK - 128, NT = KB / 64;
  using TM = RowTile<16>;  // 128-feature rows: the K main part and V
  using TR = RowTile<8>;   // 64-feature rows: the K part past 128
  static constexpr int OKM = 0, OKR = OKM + NT * TM::BYTES, OV = OKR + (DR > 0 ? NT * TR::BYTES : 0);
  static constexpr int SMEM = OV + NT * TM::BYTES;
  static_assert(DR == 0 || DR == 64, "query / key head dim 128 or 192");

  // the work unit of workgroup blockIdx.x: key u = KV head nblk_total + block, its first
  // key row k0 and the window's part [e_begin, e_end) of its list
  struct Unit {
    int kvh, e_begin, e_end;
    int64_t k0;
  };
  static __device__ __forceinline__ Unit unit(const SelFwdArgs& a) {
    Unit w;
    const int u = a.sched[blockIdx.x];
    w.kvh = u / a.nblk_total;
    const int rem = u - w.kvh * a.nblk_total;
    const int b = seq_of32(a.blkoff, a.batch, rem);
    w.k0 = a.cu_kv[b] + (int64_t)(rem - a.blkoff[b]) * a.bs;
    w.e_begin = a.nwin > 1 ? a.wofs[(int64_t)u * (a.nwin + 1) + a.win] : a.offsets[u];
    w.e_end = a.nwin > 1 ? a.wofs[(int64_t)u * (a.nwin + 1) + a.win + 1] : a.offsets[u + 1];
    return w;
  }

  template <typename T>
  static __device__ __forceinline__ void stage(const SelFwdArgs& a, const Unit& w, uint32_t smem_lds) {
    constexpr int CK = DQK / 8, CV = kDv / 8;  // 16-byte chunks per row
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);
    for (int i = threadIdx.x; i < KB * (CK + CV); i += 256) {
      const int r = i / (CK + CV), c = i - r * (CK + CV);
      const int64_t kr = (w.k0 + r) * a.n2 + w.kvh;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (c < CK) {
        if (r < a.bs) x = ldg16(k + kr * DQK + 8 * c);
        const uint32_t dst = c < 16 ? OKM + (r >> 6) * TM::BYTES + TM::off(r & 63, c)
                                    : OKR + (r >> 6) * TR::BYTES + TR::off(r & 63, c - 16);
        lds_st16_at(smem_lds + dst, x);
      } else {
        if (r < a.bs) x = ldg16(v + kr * kDv + 8 * (c - CK));
        lds_st16_at(smem_lds + OV + (r >> 6) * TM::BYTES + TM::off(r & 63, c - CK), x);
      }
    }
  }

  // S^T tile kt (keys 16 kt .. + 15 as rows, the 16 head columns of Qf) += K Q^T
  template <typename T, int NHT, int KS>
  static __device__ __forceinline__ void scores(uint32_t smem_lds, int kt, int lane,
                                                const typename Mma<T>::v8 (&Qf)[NHT][KS], f32x4 (&S)[NHT]) {
    // one lane address per part and key tile, the k-steps by XOR (the tile bases are 256-byte
    // aligned, see RowTile): kept opaque so that the compiler does not hold one register per
    // (tile, k-step) across the entry loop
    const uint32_t km = opaque(smem_lds + OKM + (kt >> 2) * TM::BYTES + 16 * (kt & 3) * TM::RB + TM::rowA(lane, 0));
    const uint32_t kr = opaque(smem_lds + OKR + (kt >> 2) * TR::BYTES + 16 * (kt & 3) * TR::RB + TR::rowA(lane, 0));
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const auto ka = s < 4 ? as_v8<T>(lds_b128_at(km ^ (64u * s))) : as_v8<T>(lds_b128_at(kr ^ (64u * (s - 4))));
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) S[ht] = Mma<T>::run(ka, Qf[ht][s], S[ht]);
    }
  }
};

// Waves per SIMD the forward's register allocation aims at: the entries' gathers are hidden
// by occupancy, so the one-head-tile 64-key form runs four (106 registers, since the LDS
// operand addresses are formed by XOR at each use instead of one register per tile and
// k-step).  The row-statistic kernel holds dY rows as well and stays at its own allocation
// (three waves, 140 registers; squeezed to four it spills and measured 2% slower).
template <int NHT, int KB>
constexpr int kv_waves() { return NHT == 1 && KB == 64 ? 4 : (NHT == 2 && KB == 128 ? 1 : 2); }

template <typename T, int DQK, int NHT, int KB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kv_waves<NHT, KB>()))) void sel_fwd_kv_kernel(
    SelFwdArgs a) {
  using V8 = typename Mma<T>::v8;
  using L = KvTiles<DQK, KB>;
  using TM = typename L::TM;
  constexpr int KS = DQK / 32, NF = kDv / 16, NKT = KB / 16;
  __shared__ __attribute__((aligned(1024))) char smem[L::SMEM];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const typename L::Unit wu = L::unit(a);
  const int kvh = wu.kvh, e_begin = wu.e_begin, e_end = wu.e_end;
  if (e_begin == e_end) return;  // whole workgroup
  const int nkt = a.bs / 16;     // key tiles of the block (bs is a multiple of 16)
  const int G = a.G;
  const T* q = static_cast<const T*>(a.q);
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  L::template stage<T>(a, wu, smem_lds);
  __syncthreads();

  // query rows of entry e (token t = list / cnt) as B operands: column = head 16 ht + l16,
  // k = features 32 s + 8 g .. + 7
  auto load_q = [&](int e, V8 (&Qf)[NHT][KS]) {
    const int ent = a.list[e];
    const int64_t t = ent / a.cnt;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int h = 16 * ht + l16;
      const int64_t row = t * a.n1 + (int64_t)kvh * G + h;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        Qf[ht][s] = as_v8<T>(h < G ? ldg16(q + row * DQK + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0));
    }
  };

  const int e_lo = (int)(a.t0 * a.cnt);  // first entry of the window
  int e = e_begin + wave;
  V8 Qc[NHT][KS];
  if (e < e_end) load_q(e, Qc);
  for (; e < e_end; e += 4) {
    V8 Qn[NHT][KS];
    if (e + 4 < e_end) load_q(e + 4, Qn);
    // S^T tiles: key tile kt holds keys 16 kt + 4 g + (0..3) of the lane's head column
    f32x4 S[NKT][NHT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) S[kt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (kt < nkt) L::template scores<T, NHT, KS>(smem_lds, kt, lane, Qc, S[kt]);
    }
    // block-local softmax per head column (log2 domain)
    float mb[NHT], lb[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
        if (kt < nkt) mx = fmaxf(mx, max4(S[kt][ht] * a.scale_log2e));
      mx = group_max(mx);
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        if (kt < nkt) {
#pragma unroll
          for (int j = 0; j < 4; ++j) S[kt][ht][j] = __builtin_amdgcn_exp2f(S[kt][ht][j] * a.scale_log2e - mx);
          sum += sum4(S[kt][ht]);
        } else {
          S[kt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      mb[ht] = mx;
      lb[ht] = group_sum(sum);
    }
    // O_b^T = V^T P^T over the block: k-step kk covers keys 32 kk .. +31 (tiles 2 kk, 2 kk + 1).
    // P^T is packed first (the scores are then dead) and the features are taken in two halves,
    // each stored as soon as it is done: fewer live registers at four waves per SIMD.
    V8 pb[NKT / 2][NHT];
#pragma unroll
    for (int kk = 0; kk < NKT / 2; ++kk)
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) pb[kk][ht] = pack8t<T>(S[2 * kk][ht], S[2 * kk + 1][ht]);
    // the entry's partial O_b / l_b as [feature tile f][head][16 features] (lane: features
    // 16 f + 4 g .. + 3 of its head), so that one store covers G x 32 contiguous bytes; m_b, l_b
    const int ent = a.list[e];
    const int64_t r = (int64_t)(ent - e_lo) * a.n2 + kvh;
    T* po = static_cast<T*>(a.part_o) + r * G * kDv;
#pragma unroll
    for (int fh = 0; fh < 2; ++fh) {
      constexpr int NFH = NF / 2;
      f32x4 O[NHT][NFH];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int f = 0; f < NFH; ++f) O[ht][f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKT / 2; ++kk) {
        if (2 * kk < nkt) {
          const uint32_t vt = opaque(smem_lds + L::OV + (kk >> 1) * TM::BYTES + 32 * (kk & 1) * TM::RB + TM::colB(lane, 0));
#pragma unroll
          for (int f = 0; f < NFH; ++f) {
            const uint32_t o = vt ^ (32u * (NFH * fh + f));
            const V8 va = __builtin_bit_cast(V8, join8(lds_tr16_at(o), lds_tr16_at(o + 16 * TM::RB)));
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) O[ht][f] = Mma<T>::run(va, pb[kk][ht], O[ht][f]);
          }
        }
      }
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        const int h = 16 * ht + l16;
        if (h < G) {
          const float inv = 1.f / lb[ht];  // <= 1: l_b includes the maximum's own term, 1
#pragma unroll
          for (int f = 0; f < NFH; ++f) {
            const uint2 w = make_uint2(pack2<T>(O[ht][f][0] * inv, O[ht][f][1] * inv),
                                       pack2<T>(O[ht][f][2] * inv, O[ht][f][3] * inv));
            *reinterpret_cast<uint2*>(po + ((NFH * fh + f) * G + h) * 16 + 4 * g) = w;
          }
          if (fh == 0 && g == 0) a.part_ml[r * G + h] = make_float2(mb[ht], lb[ht]);
        }
      }
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int s = 0; s < KS; ++s) Qc[ht][s] = Qn[ht][s];
  }
}

// The backward's row statistic without attentionOut, KV-major like the forward: per entry
// the G heads' query and dY rows are gathered as B operands, P^T = exp2(S^T scale log2 e -
// lse2) from the passed statistics, dP^T (keys x heads) = V (A: row reads of the V tile) x
// dY^T, and the entry's partial drow of each head, sum over the block's keys of P dP, is
// stored at (entry - first entry of the window) N1 + KV head G + head.
template <typename T, int DQK, int NHT, int KB>
__global__ __launch_bounds__(256) void sel_drow_kv_kernel(SelFwdArgs a) {
  using V8 = typename Mma<T>::v8;
  using L = KvTiles<DQK, KB>;
  using TM = typename L::TM;
  constexpr int KS = DQK / 32, VS = kDv / 32, NKT = KB / 16;
  __shared__ __attribute__((aligned(1024))) char smem[L::SMEM];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const typename L::Unit wu = L::unit(a);
  const int kvh = wu.kvh, e_begin = wu.e_begin, e_end = wu.e_end;
  if (e_begin == e_end) return;  // whole workgroup
  const int nkt = a.bs / 16;
  const int G = a.G;
  const T* q = static_cast<const T*>(a.q);
  const T* dy = static_cast<const T*>(a.dy);
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  L::template stage<T>(a, wu, smem_lds);
  __syncthreads();

  // query and dY rows of entry e as B operands (column = head 16 ht + l16), and lse2 per head
  auto load = [&](int e, V8 (&Qf)[NHT][KS], V8 (&Yf)[NHT][VS], float (&lse)[NHT]) {
    const int64_t t = a.list[e] / a.cnt;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int h = 16 * ht + l16;
      const int64_t row = t * a.n1 + (int64_t)kvh * G + h;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        Qf[ht][s] = as_v8<T>(h < G ? ldg16(q + row * DQK + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0));
#pragma unroll
      for (int s = 0; s < VS; ++s)
        Yf[ht][s] = as_v8<T>(h < G ? ldg16(dy + row * kDv + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0));
      lse[ht] = h < G ? a.lse2[row] : INFINITY;
    }
  };

  const int e_lo = (int)(a.t0 * a.cnt);
  int e = e_begin + wave;
  V8 Qc[NHT][KS], Yc[NHT][VS];
  float lc[NHT];
  if (e < e_end) load(e, Qc, Yc, lc);
  for (; e < e_end; e += 4) {
    V8 Qn[NHT][KS], Yn[NHT][VS];
    float ln[NHT];
    if (e + 4 < e_end) load(e + 4, Qn, Yn, ln);
    float acc[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) acc[ht] = 0.f;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      if (kt < nkt) {
        f32x4 S[NHT], D[NHT];
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) S[ht] = D[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
        L::template scores<T, NHT, KS>(smem_lds, kt, lane, Qc, S);
        const uint32_t vm = smem_lds + L::OV + (kt >> 2) * TM::BYTES + 16 * (kt & 3) * TM::RB;
#pragma unroll
        for (int s = 0; s < VS; ++s) {
          const V8 va = as_v8<T>(lds_b128_at(vm + TM::rowA(lane, s)));
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht) D[ht] = Mma<T>::run(va, Yc[ht][s], D[ht]);
        }
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[ht] += __builtin_amdgcn_exp2f(S[ht][j] * a.scale_log2e - lc[ht]) * D[ht][j];
      }
    }
    const int64_t r = (int64_t)(a.list[e] - e_lo) * a.n1 + (int64_t)kvh * G;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int h = 16 * ht + l16;
      const float d = group_sum(acc[ht]);
      if (h < G && g == 0) a.part_d[r + h] = d;
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
#pragma unroll
      for (int s = 0; s < KS; ++s) Qc[ht][s] = Qn[ht][s];
#pragma unroll
      for (int s = 0; s < VS; ++s) Yc[ht][s] = Yn[ht][s];
      lc[ht] = ln[ht];
    }
  }
}

// ndrow of each query row (token, head) of the window: minus the sum of its entries'
// partials in slot order (eight loads in flight); slots with an out-of-range id have none.
__global__ __launch_bounds__(256) void sel_drow_combine_kernel(SelFwdArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // row (t - t0) N1 + head
  if (i >= (a.t1 - a.t0) * a.n1) return;
  const int64_t tw = i / a.n1, t = a.t0 + tw;
  const int hg = (int)(i - tw * a.n1), kvh = hg / a.G;
  const int b = seq_of(a.cu_q, a.batch, t);
  const int nblk = (int)((a.cu_kv[b + 1] - a.cu_kv[b]) / a.bs);
  const int32_t* ids = a.topk + (t * a.n2 + kvh) * a.cnt;
  const float* src = a.part_d + tw * a.cnt * a.n1 + hg;  // slot sl at + sl N1
  float acc = 0.f;
  for (int s0 = 0; s0 < a.cnt; s0 += 8) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sl = s0 + j;
      const int id = sl < a.cnt ? ids[sl] : -1;
      x[j] = id >= 0 && id < nblk ? src[(int64_t)sl * a.n1] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += x[j];
  }
  a.ndrow[t * a.n1 + hg] = -acc;
}

// One wave per (token, KV head) of the window.  Lane l owns the 16-byte chunks l, l + 64,
// ... of the G x d_v block in the partials' order (chunk c: feature tile f = c / 2G, head
// (c mod 2G) / 2, features 16 f + 8 (c mod 2) .. + 7) and merges
// the slots in order with a running maximum (online softmax over the blocks); two slots per
// iteration keep eight 16-byte partial loads per lane in flight.  Slots whose id is out of
// range have no partial: one ballot per 64 slots marks the valid ones.
constexpr int kCU = 4;  // chunks per lane per pass

template <typename T>
__global__ __launch_bounds__(256) void sel_fwd_combine_kernel(SelFwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wu = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // unit within the window
  if (wu >= (a.t1 - a.t0) * a.n2) return;                           // whole wave
  const int64_t unit = a.t0 * a.n2 + wu;
  const int64_t t = unit / a.n2;
  const int kvh = (int)(unit - t * a.n2);
  const int b = seq_of(a.cu_q, a.batch, t);
  const int nblk = (int)((a.cu_kv[b + 1] - a.cu_kv[b]) / a.bs);
  uint64_t valid[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int sl = 64 * hh + lane;
    bool ok = false;
    if (sl < a.cnt) {
      const int id = a.topk[unit * a.cnt + sl];
      ok = id >= 0 && id < nblk;
    }
    valid[hh] = __ballot(ok);
  }
  auto slot_ok = [&](int sl) -> bool { return sl < a.cnt && ((valid[sl >> 6] >> (sl & 63)) & 1); };
  const int G = a.G, chunks = G * (kDv / 8);
  const int64_t r0 = (t - a.t0) * a.cnt;  // the token's first entry in the window
  const T* po = static_cast<const T*>(a.part_o);
  for (int c0 = lane; c0 < chunks; c0 += 64 * kCU) {
    float acc[kCU][8], m[kCU], l[kCU];
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
      m[u] = -INFINITY;
      l[u] = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[u][j] = 0.f;
    }
    for (int sl = 0; sl < a.cnt; sl += 2) {
      uint4 x[2][kCU];
      float2 ml[2][kCU];
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const bool ok = slot_ok(sl + d);
        const int64_t r = ((r0 + sl + d) * a.n2 + kvh) * G;  // (entry, head 0) row
#pragma unroll
        for (int u = 0; u < kCU; ++u) {
          const int c = c0 + 64 * u;
          x[d][u] = make_uint4(0, 0, 0, 0);
          ml[d][u] = make_float2(-INFINITY, 0.f);
          if (ok && c < chunks) {
            x[d][u] = ldg16_stream(po + r * kDv + 8 * c);
            ml[d][u] = a.part_ml[r + (c % (2 * G)) / 2];
          }
        }
      }
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        if (!slot_ok(sl + d)) continue;
#pragma unroll
        for (int u = 0; u < kCU; ++u) {
          const float mn = fmaxf(m[u], ml[d][u].x);
          const float sc = __builtin_amdgcn_exp2f(m[u] - mn);  // 0 before the first valid slot
          const float w = ml[d][u].y * __builtin_amdgcn_exp2f(ml[d][u].x - mn);
          const uint32_t xs[4] = {x[d][u].x, x[d][u].y, x[d][u].z, x[d][u].w};
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            acc[u][2 * q2] = acc[u][2 * q2] * sc + w * t2f<T>((uint16_t)(xs[q2] & 0xffffu));
            acc[u][2 * q2 + 1] = acc[u][2 * q2 + 1] * sc + w * t2f<T>((uint16_t)(xs[q2] >> 16));
          }
          l[u] = l[u] * sc + w;
          m[u] = mn;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
      const int c = c0 + 64 * u;
      if (c >= chunks) continue;
      const int f = c / (2 * G), h = (c % (2 * G)) / 2, half = c & 1;
      const float inv = l[u] > 0.f ? 1.f / l[u] : 0.f;
      const int64_t row = t * a.n1 + (int64_t)kvh * G + h;
      const uint4 y = make_uint4(pack2<T>(acc[u][0] * inv, acc[u][1] * inv), pack2<T>(acc[u][2] * inv, acc[u][3] * inv),
                                 pack2<T>(acc[u][4] * inv, acc[u][5] * inv), pack2<T>(acc[u][6] * inv, acc[u][7] * inv));
      sts16_stream(static_cast<T*>(a.o) + row * kDv + 16 * f + 8 * half, y);
      if (f == 0 && half == 0) {
        // statistics in natural units: m = m2 ln 2, l as summed; no valid block: -inf, 0
        const float mn = l[u] > 0.f ? m[u] * 0.6931471805599453f : -INFINITY;
        const float lv = l[u];
        *reinterpret_cast<f32x4*>(a.smax + row * 8) = f32x4{mn, mn, mn, mn};
        *reinterpret_cast<f32x4*>(a.smax + row * 8 + 4) = f32x4{mn, mn, mn, mn};
        *reinterpret_cast<f32x4*>(a.ssum + row * 8) = f32x4{lv, lv, lv, lv};
        *reinterpret_cast<f32x4*>(a.ssum + row * 8 + 4) = f32x4{lv, lv, lv, lv};
      }
    }
  }
}

template <typename T, bool DROW>
hipError_t launch_kv_t(const SelFwdArgs& a, hipStream_t s) {
  const int nkeys = a.n2 * a.nblk_total;
  if (nkeys == 0) return hipSuccess;
  const dim3 grid((unsigned)nkeys), block(256);
  const bool two = a.G > 16, wide = a.bs > 64;
#define AB_KV(DQK, NHT, KB)                                                                           \
  do {                                                                                                \
    if (DROW) hipLaunchKernelGGL((sel_drow_kv_kernel<T, DQK, NHT, KB>), grid, block, 0, s, a);        \
    else hipLaunchKernelGGL((sel_fwd_kv_kernel<T, DQK, NHT, KB>), grid, block, 0, s, a);              \
  } while (0)
#define AB_KV_D(DQK)                                                                                  \
  do {                                                                                                \
    if (two) {                                                                                        \
      if (wide) AB_KV(DQK, 2, 128);                                                                   \
      else AB_KV(DQK, 2, 64);                                                                         \
    } else {                                                                                          \
      if (wide) AB_KV(DQK, 1, 128);                                                                   \
      else AB_KV(DQK, 1, 64);                                                                         \
    }                                                                                                 \
  } while (0)
  if (a.d_qk == 192) AB_KV_D(192);
  else AB_KV_D(128);
#undef AB_KV_D
#undef AB_KV
  return hipGetLastError();
}

template <typename T>
hipError_t launch_combine_t(const SelFwdArgs& a, hipStream_t s) {
  const int64_t units = (a.t1 - a.t0) * a.n2;
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL(sel_fwd_combine_kernel<T>, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_selected_forward_kv(const SelFwdArgs& a, hipStream_t s) {
  if (!selected_supported(a.d_qk, a.d_v, a.G, a.bs)) return hipErrorInvalidValue;
  return a.is_f16 ? launch_kv_t<_Float16, false>(a, s) : launch_kv_t<__bf16, false>(a, s);
}

hipError_t launch_selected_drow_kv(const SelFwdArgs& a, hipStream_t s) {
  if (!selected_supported(a.d_qk, a.d_v, a.G, a.bs)) return hipErrorInvalidValue;
  return a.is_f16 ? launch_kv_t<_Float16, true>(a, s) : launch_kv_t<__bf16, true>(a, s);
}

hipError_t launch_selected_drow_combine(const SelFwdArgs& a, hipStream_t s) {
  const int64_t rows = (a.t1 - a.t0) * a.n1;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(sel_drow_combine_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_selected_forward_combine(const SelFwdArgs& a, hipStream_t s) {
  return a.is_f16 ? launch_combine_t<_Float16>(a, s) : launch_combine_t<__bf16>(a, s);
}

}  // namespace ab
