// Lightning-indexer backward (page "aclnnLightningIndexerGrad", formula section):
//   S  = ReLU(Q . Gather(K, Indices))          per query token t, key head n2, selected key k
//   Y  = dy * Weights                          Y[t, h, k] = dy[t, n2, k] W[t, h]
//   dW = Reduce(S * dy)                        dW[t, h] = sum_k S[t, h, k] dy[t, n2, k]
//   dQ = ReluGrad(Y, S) . Gather(K, Indices)   R = Y where S > 0, else 0
//   dK = ScatterAdd(ReluGrad(Y, S) . Q, Indices)
// for the G = N1 / N2 query heads h of key head n2.
//
// Query-major: one workgroup (4 waves) per (token, key head).  The G heads are the columns
// of the MFMA tiles (G padded to 16, 32 or 64; padding heads carry zero weights), and the
// topK selected keys pass in chunks of 64, 16 per wave:
//   S^T (keys x heads)  = K (A: the wave's 16 gathered key rows, 16 bytes per lane straight
//                         from global memory) x Q^T (B: the head rows, resident);
//   R^T                 = where(S^T > 0, dy W, 0); dW += S^T dy per head (lane);
//   dQ^T (feat x heads) += K^T (A: column reads of the key rows, staged in LDS) x R^T (B: read
//                         back from LDS), each wave over its quarter of the features and all
//                         64 keys of the chunk, 16 (one wave's) per k-step;
//   C^T (feat x keys)   = Q^T (A: column reads of the Q tile in LDS) x R (B: column reads of
//                         R^T written to LDS as [head][key]);  C is the key rows' share of dK.
// C goes either, row by row, to a share buffer indexed by (token, key head, slot), rounded
// to bf16, that a second kernel sums in fp32 over each key's inverted-index list in
// ascending order (deterministic; the default), or to an fp32 accumulator with atomics.  The
// next chunk's key rows, ids and dy load while a chunk computes.  dQ (each wave its own
// features) and dW (the four waves' sums added in LDS) have one writer each.  An
// out-of-range index contributes nothing and raises the flag.
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

constexpr int kIdxD = 128;    // head dim
constexpr int kIdxChunk = 64; // keys per chunk (16 per wave)

__device__ __forceinline__ float group_sum4(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <int NHT, bool ATOMIC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void idx_bwd_kernel(IdxArgs a) {
  constexpr int D = kIdxD, KS = D / 32;
  constexpr int NFQ = D / 64;                  // dQ feature tiles of a wave: features 32 w .. + 31
  constexpr int GP = 16 * NHT;                 // padded head count
  using TQ = RowTile<D / 8>;                   // Q tile / key sub-tiles: rows of 256 bytes
  constexpr int OQ = 0;                        // Q tile: GP rows (64-row tile)
  constexpr int OK = TQ::BYTES;                // key rows: 4 waves x 16 rows (one 64-row tile)
  constexpr int OR = OK + TQ::BYTES;           // R^T as [head][16 keys] bf16 per wave: GP x 32 bytes
  constexpr int RB = GP * 32;
  constexpr int SMEM = OR + 4 * RB;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t unit = a.unit0 + blockIdx.x;     // (token, key head)
  const int64_t t = unit / a.n2;
  const int kvh = (int)(unit - t * a.n2);
  const int b = seq_of(a.cu_q, a.batch, t);
  const int64_t kv0 = a.cu_kv[b];
  const int S2 = (int)(a.cu_kv[b + 1] - kv0);
  const int G = a.G;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* wts = static_cast<const uint16_t*>(a.weights);
  const uint16_t* dyp = static_cast<const uint16_t*>(a.dy);
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  const int64_t qrow0 = t * a.n1 + (int64_t)kvh * G;  // first query head of the group

  // Q tile in LDS (rows = heads, zero rows for padding heads): the B operands of S^T (row
  // reads) and the A operands of C^T (column reads)
  for (int i = tid; i < GP * (D / 8); i += 256) {
    const int r = i / (D / 8), c = i % (D / 8);
    uint4 x = make_uint4(0, 0, 0, 0);
    if (r < G) x = ldg16(q + (qrow0 + r) * D + 8 * c);
    lds_st16_at(smem_lds + OQ + TQ::off(r, c), x);
  }
  float wv[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = 16 * ht + l16;
    wv[ht] = h < G ? bf2f(wts[qrow0 + h]) : 0.f;
  }
  // dQ^T of this wave's features 32 w .. + 31 (tiles 2 w, 2 w + 1) over every key of the chunk
  f32x4 dQ[NFQ][NHT];
#pragma unroll
  for (int f = 0; f < NFQ; ++f)
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) dQ[f][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dW[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) dW[ht] = 0.f;

  const uint32_t ksub = smem_lds + OK + 16 * w * TQ::RB;    // this wave's 16 key rows
  const uint32_t rt = smem_lds + OR + w * RB;               // this wave's R^T [head][key]
  const int32_t* ids = a.indices + unit * a.topk;
  const uint16_t* dyrow = dyp + unit * a.topk;

  // the gathered inputs of chunk c0: this lane's key row (slot c0 + 16 w + l16) 16 bytes per
  // k-step, and dy of the keys 4 g .. 4 g + 3 of the wave's 16 (the rows of its S^T values)
  struct ChunkIn {
    uint4 kx[KS];
    float dyk[4];
    int id;
  };
  auto load_chunk = [&](int c0, ChunkIn& in) {
    const int slot = c0 + 16 * w + l16;
    in.id = slot < a.topk ? ids[slot] : -1;
    const bool kvalid = slot < a.topk && in.id >= 0 && in.id < S2;
    const int64_t krow = (kv0 + (kvalid ? in.id : 0)) * a.n2 + kvh;
#pragma unroll
    for (int s = 0; s < KS; ++s) in.kx[s] = kvalid ? ldg16(k + krow * D + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sl = c0 + 16 * w + 4 * g + j;
      in.dyk[j] = sl < a.topk ? bf2f(dyrow[sl]) : 0.f;
    }
  };
  ChunkIn cur;
  load_chunk(0, cur);
  __syncthreads();  // Q tile in LDS

  for (int c0 = 0; c0 < a.topk; c0 += kIdxChunk) {
    const int slot = c0 + 16 * w + l16;
    const bool kvalid = slot < a.topk && cur.id >= 0 && cur.id < S2;
    if (slot < a.topk && !kvalid && a.flag) a.flag[0] = 1;
    // key rows into LDS: lane (l16, g) holds chunks 4 s + g of key row l16
#pragma unroll
    for (int s = 0; s < KS; ++s) lds_st16_at(ksub + TQ::off(l16, 4 * s + g), cur.kx[s]);
    // S^T = K Q^T
    f32x4 St[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc = mfma_16x16x32(__builtin_bit_cast(bf16x8, cur.kx[s]),
                            lds_b128_at(smem_lds + OQ + 16 * ht * TQ::RB + TQ::rowA(lane, s)), acc);
      St[ht] = acc;
    }
    // R^T, dW, and R^T -> LDS as [head][key] (8 bytes: keys 4 g .. + 3 of head 16 ht + l16)
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f32x4 r;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sv = St[ht][j];
        dW[ht] += fmaxf(sv, 0.f) * cur.dyk[j];
        r[j] = sv > 0.f ? cur.dyk[j] * wv[ht] : 0.f;
      }
      *reinterpret_cast<__attribute__((address_space(3))) i16x4*>((uintptr_t)(rt + (16 * ht + l16) * 32 + 8 * g)) = pack4(r);
    }
    // the next chunk's inputs load while this one computes
    ChunkIn nxt;
    if (c0 + kIdxChunk < a.topk) load_chunk(c0 + kIdxChunk, nxt);
    __syncthreads();  // every wave's key rows and R^T in LDS
    // dQ^T (features 32 w .. + 31) += K^T R^T over the 64 keys, 16 (one wave's) per k-step
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      i16x4 rb[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
        rb[ht] = *reinterpret_cast<const __attribute__((address_space(3))) i16x4*>(
            (uintptr_t)(smem_lds + OR + ks * RB + (16 * ht + l16) * 32 + 8 * g));
#pragma unroll
      for (int f = 0; f < NFQ; ++f) {
        const i16x4 kt = lds_tr16_at(smem_lds + OK + 16 * ks * TQ::RB + TQ::colB(lane, NFQ * w + f));
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) dQ[f][ht] = mfma_16x16x16(kt, rb[ht], dQ[f][ht]);
      }
    }
    __syncthreads();  // every wave is done with the key rows and R^T of this chunk
    // C^T = Q^T R (k = heads, 16 per step): this wave's 16 keys' shares of dK
    i16x4 rk[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) rk[ht] = lds_tr16_at(rt + (16 * ht + 4 * g + (l16 >> 2)) * 32 + 8 * (l16 & 3));
    // The C tiles go out through this wave's key-row slot of LDS (4 KiB, free now that every
    // wave's dQ product has read it), 64 features at a time as [16 keys][16 chunks of 16 B]
    // with chunk c of row r at c ^ r, so that every global store or atomic covers whole key
    // rows instead of 16 rows x 64 bytes.  C tile of feature tile f: lane holds key l16 of
    // the wave, features 16 f + 4 g + (0..3).
    const int cid = cur.id;
    const int cvalid = kvalid;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int f4 = 0; f4 < 4; ++f4) {
        const int f = 4 * hf + f4;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
          acc = mfma_16x16x16(lds_tr16_at(smem_lds + OQ + 16 * ht * TQ::RB + TQ::colB(lane, f)), rk[ht], acc);
        lds_st16_at(ksub + l16 * 256 + 16 * ((4 * f4 + g) ^ l16), __builtin_bit_cast(uint4, acc));
      }
      if constexpr (ATOMIC) {
        // one key row per instruction: lane = feature 64 hf + lane
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rid = __shfl(cid, r);
          const float v = lds_f32_at(ksub + r * 256 + 16 * ((lane >> 2) ^ r) + 4 * (lane & 3));
          if (__shfl(cvalid, r)) atomicAdd(a.dk_acc + ((kv0 + rid) * a.n2 + kvh) * D + 64 * hf + lane, v);
        }
      } else {
        // four key rows per instruction: lane = row 4 i + lane / 16, chunk lane % 16; the
        // share leaves as bf16 (8 bytes per lane, 128 contiguous bytes per row half)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * i + (lane >> 4), c = lane & 15;
          const f32x4 v = lds_f32x4_at(ksub + r * 256 + 16 * (c ^ r));
          const int sl = c0 + 16 * w + r;
          if (sl < a.topk) {
            const u32x2 x = {(uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16),
                             (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16)};
            __builtin_nontemporal_store(x, reinterpret_cast<u32x2*>(a.contrib + ((unit - a.unit0) * a.topk + sl) * D + 64 * hf + 4 * c));
          }
        }
      }
    }
    asm volatile("" ::: "memory");  // this chunk's LDS reads come before the next chunk's writes
    cur = nxt;
  }

  // ---- dW: per head, over the lane groups and the four waves (in the Q tile's space, once
  // every wave has done its last C^T product) ----
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const float sv = group_sum4(dW[ht]);
    if (g == 0) red[w * GP + 16 * ht + l16] = sv;
  }
  __syncthreads();
  if (tid < G) {
    const float sv = (red[tid] + red[GP + tid]) + (red[2 * GP + tid] + red[3 * GP + tid]);
    static_cast<uint16_t*>(a.dweights)[qrow0 + tid] = f2bf(sv);
  }
  // ---- dQ: this wave's features, every head; lane holds head 16 ht + l16, features
  // 32 w + 16 f + 4 g + (0..3) ----
  uint16_t* dq = static_cast<uint16_t*>(a.dq);
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = 16 * ht + l16;
    if (h >= G) continue;
#pragma unroll
    for (int f = 0; f < NFQ; ++f) {
      const f32x4 v = dQ[f][ht];
      const uint2 o = make_uint2((uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16),
                                 (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16));
      *reinterpret_cast<uint2*>(dq + (qrow0 + h) * D + 16 * (NFQ * w + f) + 4 * g) = o;
    }
  }
}

// Deterministic dK: one wave per key row (token j, key head); its list holds the entries
// t topK + slot that selected it, ascending; the window's entries are added in that order to
// the fp32 accumulator (two features per lane).
__global__ __launch_bounds__(256) void idx_dk_reduce_kernel(IdxArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t key = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (key >= a.nkeys) return;  // whole wave
  const int kvh = (int)(key / a.T2);
  const int64_t j = key - (int64_t)kvh * a.T2;
  const int e0 = a.nwin > 1 ? a.wofs[key * (a.nwin + 1) + a.win] : a.offsets[key];
  const int e1 = a.nwin > 1 ? a.wofs[key * (a.nwin + 1) + a.win + 1] : a.offsets[key + 1];
  if (e0 == e1) return;
  float2 acc = *reinterpret_cast<const float2*>(a.dk_acc + (j * a.n2 + kvh) * kIdxD + 2 * lane);
  // the share of list entry `ent` (t topK + slot): read once, so not kept in the caches
  auto share = [&](int ent) {
    const int64_t t = ent / a.topk, slot = ent - t * a.topk;
    const int64_t u = t * a.n2 + kvh - a.unit0;
    const uint32_t x = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a.contrib + (u * a.topk + slot) * kIdxD + 2 * lane));
    return f32x2{bf2f((uint16_t)(x & 0xffffu)), bf2f((uint16_t)(x >> 16))};
  };
  int e = e0;
  for (; e + 16 <= e1; e += 16) {  // sixteen loads in flight, added in list order
    f32x2 c[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = share(a.list[e + i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc.x += c[i][0];
      acc.y += c[i][1];
    }
  }
  for (; e < e1; ++e) {
    const f32x2 c = share(a.list[e]);
    acc.x += c[0];
    acc.y += c[1];
  }
  *reinterpret_cast<float2*>(a.dk_acc + (j * a.n2 + kvh) * kIdxD + 2 * lane) = acc;
}

__global__ __launch_bounds__(256) void idx_dk_cast_kernel(const float* acc, uint16_t* dk, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) dk[i] = f2bf(acc[i]);
}

__global__ __launch_bounds__(256) void idx_zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

unsigned grid_of(int64_t n, int64_t per) {
  int64_t g = (n + per - 1) / per;
  return (unsigned)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

}  // namespace

bool indexer_supported(int d, int G) { return d == kIdxD && G >= 1 && G <= 64; }

hipError_t launch_indexer_zero(const IdxArgs& a, hipStream_t s) {
  const int64_t n = a.T2 * a.n2 * kIdxD;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(idx_zero_kernel, dim3(grid_of(n, 256)), dim3(256), 0, s, a.dk_acc, n);
  return hipGetLastError();
}

hipError_t launch_indexer_qm(const IdxArgs& a, hipStream_t s) {
  const int64_t units = a.unit1 - a.unit0;
  if (units <= 0) return hipSuccess;
  if (!indexer_supported(a.d, a.G)) return hipErrorInvalidValue;
  const IdxArgs& k = a;  // workgroup i takes unit unit0 + i
  const dim3 grid((unsigned)units), block(256);
  const int nht = a.G <= 16 ? 1 : (a.G <= 32 ? 2 : 4);
#define AB_IDX(NHT)                                                                                            \
  do {                                                                                                         \
    if (a.atomic) hipLaunchKernelGGL((idx_bwd_kernel<NHT, true>), grid, block, 0, s, k);                       \
    else hipLaunchKernelGGL((idx_bwd_kernel<NHT, false>), grid, block, 0, s, k);                               \
  } while (0)
  if (nht == 1) AB_IDX(1);
  else if (nht == 2) AB_IDX(2);
  else AB_IDX(4);
#undef AB_IDX
  return hipGetLastError();
}

hipError_t launch_indexer_dk_reduce(const IdxArgs& a, hipStream_t s) {
  if (a.nkeys == 0) return hipSuccess;
  hipLaunchKernelGGL(idx_dk_reduce_kernel, dim3(grid_of(a.nkeys, 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_indexer_dk_cast(const IdxArgs& a, hipStream_t s) {
  const int64_t n = a.T2 * a.n2 * kIdxD;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(idx_dk_cast_kernel, dim3(grid_of(n, 256)), dim3(256), 0, s, (const float*)a.dk_acc,
                     (uint16_t*)a.dk, n);
  return hipGetLastError();
}

}  // namespace ab
