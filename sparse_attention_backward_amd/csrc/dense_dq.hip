// Dense dQ from the stored dS tiles: dQ = scale * dS K (bf16 MFMA, fp32 accumulation).
//
// Page "aclnnFlashAttentionUnpaddingScoreGradV3", Formula section: dQ = dS K / sqrt(d),
// dqRope = dS kRope / sqrt(d), with K = [key, keyRope].  dS itself comes from the KV-major
// kernel, which leaves one transposed 64 x 64 bf16 block per (query tile, key tile, head)
// in the workspace; this kernel is then a plain product, with no recomputation of S or dP.
//
// One workgroup (4 waves) owns a 64-row query tile of HP query heads that share a KV head
// (all G heads, in passes of HP).  Per key tile it stages the K tile and the HP dS^T blocks
// in LDS (double buffered, global->LDS transfers one tile ahead) and accumulates
// dQ += dS K.  The waves form a 2 x 2 grid: rows 32(w>>1) .. +31 and feature columns
// (DQK/2)(w&1) .. of every head.  Both operands are read with ds_read_b64_tr_b16: the
// contraction runs over keys, which are the rows of both staged tiles.  Keys are taken
// in the order {4g + j, 16 + 4g + j} on both sides, which keeps the reads conflict free.
// Fixed loop order, no atomics: deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

constexpr int kT = 64;           // rows per query tile, keys per key tile
constexpr int kCB = 1024 + 128;  // bytes per chunk column of a staged 64-row tile
typedef __attribute__((address_space(3))) void lds_void;

struct DqArgs {
  const uint16_t* k; const uint16_t* k_rope;
  const uint16_t* ds;           // [block][head][64 keys][64 rows]
  uint16_t* dq; uint16_t* dq_rope;
  const int64_t* cu_q; const int64_t* cu_kv;
  const int64_t* ds_base;       // [B + 1]
  const int32_t* tiles;         // [n][2] (sequence, query tile)
  int n1, n2, G, d_main, d_rope;
  int causal;
  float scale;
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

template <int MOFF, int OFF>
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%3"
               ::"v"(src), "s"(lds), "i"(MOFF), "i"(OFF) : "memory", "m0", "scc");
}

template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

template <int DQK, int HP>
__global__ __launch_bounds__(256, 1) void dense_dq_ds_kernel(DqArgs a) {
  constexpr int NQ = DQK / 16, NF = NQ / 2;   // feature tiles in total / per wave
  constexpr int QCH = DQK / 8;                // 16-byte chunks per K row
  constexpr int KLD = QCH / 4;                // K transfer instructions per wave
  constexpr int DLD = 2 * HP;                 // dS transfer instructions per wave (8 chunks per block)
  constexpr int KB = QCH * kCB, DB = 8 * kCB;
  constexpr int SB = KB + HP * DB;            // one stage
  static_assert(2 * SB <= 160 * 1024, "two stages must fit in LDS");
  static_assert(HP * (KB + 0) <= 2 * SB, "output tiles must fit");
  __shared__ __attribute__((aligned(16))) char smem[2 * SB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fh = w & 1, rh = w >> 1;
  const int l16 = lane & 15, g = lane >> 4, jj = l16 >> 2, qq = l16 & 3;

  const int b = a.tiles[2 * blockIdx.x], qt = a.tiles[2 * blockIdx.x + 1];
  const int kvh = blockIdx.y;
  const int64_t qs = a.cu_q[b], ks = a.cu_kv[b];
  const int S1 = (int)(a.cu_q[b + 1] - qs), S2 = (int)(a.cu_kv[b + 1] - ks);
  const int nkt = (S2 + kT - 1) / kT;
  const int nkt_run = a.causal ? min(qt + 1, nkt) : nkt;
  const int nvalid = min(kT, S1 - qt * kT);
  const int qmain = a.d_main / 8;
  const int64_t blk0 = a.ds_base[b];

  // per-lane LDS offset of a column read: keys 4g + jj (+16, +32 ks), chunk qq/2, half qq&1
  const int colb = (qq >> 1) * kCB + 16 * (4 * g + jj) + 8 * (qq & 1);
  const int kq = (qmain - w + 3) >> 2;  // K chunks k < kq come from `key`, the rest from keyRope
  const uint32_t smem_lds = lds_addr(smem);

  for (int hp0 = 0; hp0 < a.G; hp0 += HP) {
    const int h0 = kvh * a.G + hp0;  // first query head of this pass

    // issue(): K tile (chunks w + 4k, lane = key) and the HP dS^T blocks (chunks w, w + 4)
    auto issue = [&](int kt, int soff) {
      const int nk = min(kT, S2 - kt * kT);
      const int64_t kr = (ks + (int64_t)kt * kT + min(lane, nk - 1)) * a.n2 + kvh;
      const char* krow = reinterpret_cast<const char*>(a.k + kr * a.d_main) + 16 * w;
      const char* rrow = reinterpret_cast<const char*>(a.k_rope + kr * a.d_rope) + 16 * (w - qmain);
      const uint32_t kb = smem_lds + soff + w * kCB;
      static_for<KLD>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        dma16<k * (4 * kCB - 64), 64 * k>(k < kq ? krow : rrow, kb);
      });
      const int64_t blk = blk0 + (a.causal ? (int64_t)qt * (qt + 1) / 2 + kt : (int64_t)qt * nkt + kt);
      const char* drow = reinterpret_cast<const char*>(a.ds + ((blk * a.n1 + h0) * (kT * kT) + lane * kT)) + 16 * w;
      static_for<HP>([&](auto hc) {
        constexpr int hh = decltype(hc)::value;
        const uint32_t db = smem_lds + soff + KB + hh * DB + w * kCB;
        // chunks w and w + 4 of key row `lane` of head h0 + hh (block rows are 128 bytes)
        dma16<0, 0>(drow + hh * (kT * kT * 2), db);
        dma16<4 * kCB - 64, 64>(drow + hh * (kT * kT * 2), db);
      });
    };

    f32x4 acc[HP][2][NF];
#pragma unroll
    for (int hh = 0; hh < HP; ++hh)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[hh][rt][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto colfrag = [&](const char* base, int chunk, int ks2) -> bf16x8 {
      const int o = colb + chunk * kCB + 512 * ks2;
      return join8(lds_read_tr16(reinterpret_cast<const uint16_t*>(base + o)),
                   lds_read_tr16(reinterpret_cast<const uint16_t*>(base + o + 256)));
    };

    __syncthreads();  // the previous pass's output tiles have been read
    if (nkt_run > 0) issue(0, 0);
    for (int kt = 0; kt < nkt_run; ++kt) {
      wait_vmcnt<0>();
      barrier_no_vm_wait();  // tile kt is in LDS; the other stage is free
      const char* cur = smem + (kt & 1) * SB;
      if (kt + 1 < nkt_run) issue(kt + 1, (~kt & 1) * SB);
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        bf16x8 kb[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f) kb[f] = colfrag(cur, 2 * (fh * NF + f), ks2);
#pragma unroll
        for (int hh = 0; hh < HP; ++hh) {
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            const bf16x8 da = colfrag(cur + KB + hh * DB, 2 * (2 * rh + rt), ks2);
#pragma unroll
            for (int f = 0; f < NF; ++f) acc[hh][rt][f] = mfma_16x16x32(da, kb[f], acc[hh][rt][f]);
          }
        }
      }
    }

    // ---- epilogue: bf16 through LDS (chunk-major [chunk][64 rows] per head), 16-byte stores
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < HP; ++hh) {
      uint16_t* O = reinterpret_cast<uint16_t*>(smem + hh * KB);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 32 * rh + 16 * rt + 4 * g + i, col = 16 * (fh * NF + f) + l16;
            O[((col >> 3) * kCB + 16 * r) / 2 + (col & 7)] = f2bf(acc[hh][rt][f][i] * a.scale);
          }
    }
    __syncthreads();
    for (int idx = tid; idx < HP * kT * QCH; idx += 256) {
      const int hh = idx / (kT * QCH), rem = idx - hh * (kT * QCH);
      const int r = rem / QCH, c = rem - r * QCH, d = 8 * c;
      if (r < nvalid) {
        const int64_t qr = (qs + (int64_t)qt * kT + r) * a.n1 + h0 + hh;
        uint16_t* dst = d < a.d_main ? a.dq + qr * a.d_main + d : a.dq_rope + qr * a.d_rope + (d - a.d_main);
        sts16(dst, *reinterpret_cast<const uint4*>(smem + hh * KB + c * kCB + 16 * r));
      }
    }
  }
}

template <int DQK>
hipError_t launch_hp(const DqArgs& k, int G, dim3 grid, hipStream_t s) {
  if (G % 4 == 0) hipLaunchKernelGGL((dense_dq_ds_kernel<DQK, 4>), grid, dim3(256), 0, s, k);
  else if (G % 2 == 0) hipLaunchKernelGGL((dense_dq_ds_kernel<DQK, 2>), grid, dim3(256), 0, s, k);
  else hipLaunchKernelGGL((dense_dq_ds_kernel<DQK, 1>), grid, dim3(256), 0, s, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_dq_from_ds(const DenseArgs& a, hipStream_t s) {
  if (a.n_q_tiles == 0) return hipSuccess;
  DqArgs k{};
  k.k = (const uint16_t*)a.k; k.k_rope = (const uint16_t*)a.k_rope;
  k.ds = (const uint16_t*)a.ds;
  k.dq = (uint16_t*)a.dq; k.dq_rope = (uint16_t*)a.dq_rope;
  k.cu_q = a.cu_q; k.cu_kv = a.cu_kv; k.ds_base = a.ds_base; k.tiles = a.q_tiles;
  k.n1 = a.n1; k.n2 = a.n2; k.G = a.G;
  k.d_main = a.d_main; k.d_rope = a.d_rope;
  k.causal = a.causal; k.scale = a.scale;
  const dim3 grid(a.n_q_tiles, a.n2);
  const int dqk = a.d_main + a.d_rope;
  if (dqk == 192) return launch_hp<192>(k, a.G, grid, s);
  if (dqk == 128) return launch_hp<128>(k, a.G, grid, s);
  if (dqk == 64) return launch_hp<64>(k, a.G, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace ab
