// Selected (NSA) attention, query-major passes over the gathered key / value rows:
//
//   forward  (page "NsaSelectedAttentionGrad": the backward consumes the forward's
//            attentionOut, softmaxMax and softmaxSum, "intermediate outputs of the forward"):
//            for every query token t and KV head, its G query heads attend to the
//            selectedBlockCount blocks of selectedBlockSize rows that topkIndices[t, kvh]
//            gathers (selectedKey = Gather(key, ids), selectedValue = Gather(value, ids)):
//              s = scale Q K^T,  m = max s,  l = sum exp(s - m),  O = sum exp(s - m) V / l,
//            with softmaxMax = m and softmaxSum = l written to all 8 lanes of [T1, N1, 8].
//   row statistic without attentionOut (the same page lists attentionOut as optional):
//              drow = sum_j P_j dP_j over the gathered rows, P_j = exp(s_j - m) / l from the
//              passed statistics and dP = dY V^T; stored negated (ndrow) for the backward.
//
// One wave per (token, KV head); the four waves of a workgroup are independent.  The G
// query heads are the columns of the MFMA tiles (one 16-column tile for G <= 16, two for
// G <= 32), so every product is computed transposed:
//   S^T (keys x heads)     = K (A: a 16 x 32 slice of 16 key rows, read from global memory
//                            16 bytes per lane) x Q^T (B: the head rows, resident);
//   O^T (features x heads) = V^T (A: column reads of the value rows, staged in LDS) x P^T
//                            (B: two S^T tiles of consecutive keys packed as 8 k values);
//   dP^T (keys x heads)    = V (A, like K) x dY^T (B, resident).
// The lane that holds column h of a C tile holds head h: the row maximum and sum of a head
// are reduced over the lane's 4 values, across its 4 lane groups and over the key tiles.
// Keys are taken in chunks of up to 64 (one LDS value tile of 64 rows); the softmax of the
// forward is formed online chunk by chunk in the log2 domain (exp2 of s scale log2 e).
// An out-of-range id is skipped (its block contributes nothing) and raises the flag.
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

template <typename T>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (T)x) | ((uint32_t)__builtin_bit_cast(uint16_t, (T)y) << 16);
}

__device__ __forceinline__ float max4(f32x4 v) { return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])); }
__device__ __forceinline__ float sum4(f32x4 v) { return (v[0] + v[1]) + (v[2] + v[3]); }
// Reduce across the four lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48 hold one head).
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

constexpr int kChunk = 64;  // keys per LDS value tile

template <typename T, int DQK, int DV, int NHT, bool DROW>
__global__ __launch_bounds__(256) void sel_fwd_kernel(SelFwdArgs a) {
  using V8 = typename Mma<T>::v8;
  constexpr int KS = DQK / 32, VS = DV / 32, NF = DV / 16;
  using TV = RowTile<DV / 8>;  // value tile: 64 rows of DV elements
  __shared__ __attribute__((aligned(1024))) char smem[DROW ? 16 : 4 * TV::BYTES];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t unit = (int64_t)blockIdx.x * 4 + wave;
  if (unit >= a.T1 * a.n2) return;  // whole wave; the waves never synchronise
  const int64_t t = unit / a.n2;
  const int kvh = (int)(unit - t * a.n2);
  const int b = seq_of(a.cu_q, a.batch, t);
  const int64_t kv0 = a.cu_kv[b];
  const int nblk = (int)((a.cu_kv[b + 1] - kv0) / a.bs);
  const int G = a.G;
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);

  // Q^T (and dY^T) as B operands: lane column = head 16 ht + l16, k = features 32 s + 8 g ..
  V8 Qf[NHT][KS];
  V8 Yf[NHT][DROW ? VS : 1];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = 16 * ht + l16;
    const int64_t row = t * a.n1 + (int64_t)kvh * G + h;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      Qf[ht][s] = as_v8<T>(h < G ? ldg16(q + row * DQK + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0));
    if constexpr (DROW) {
      const T* dy = static_cast<const T*>(a.dy);
#pragma unroll
      for (int s = 0; s < VS; ++s)
        Yf[ht][s] = as_v8<T>(h < G ? ldg16(dy + row * DV + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0));
    }
  }
  // per head (lane column): running maximum (log2 domain), sum, and (forward) O^T tiles;
  // row statistic mode: lse2 of the head and the running sum of P dP
  float mrun[NHT], lrun[NHT], lse[NHT];
  f32x4 O[NHT][NF];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    mrun[ht] = -INFINITY;
    lrun[ht] = 0.f;
    lse[ht] = 0.f;
    if constexpr (DROW) {
      const int h = 16 * ht + l16;
      lse[ht] = h < G ? a.lse2[t * a.n1 + (int64_t)kvh * G + h] : INFINITY;
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) O[ht][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t vt = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(smem + wave * TV::BYTES);
  const int32_t* ids = a.topk + unit * a.cnt;

  for (int i = 0; i < a.cnt; ++i) {
    const int id = __builtin_amdgcn_readfirstlane(ids[i]);
    if (id < 0 || id >= nblk) {
      if (a.flag && lane == 0) a.flag[0] = 1;
      continue;
    }
    const int64_t r0 = kv0 + (int64_t)id * a.bs;
    for (int c0 = 0; c0 < a.bs; c0 += kChunk) {
      const int ck = min(kChunk, a.bs - c0);  // keys of this chunk, a multiple of 16
      const int nkt = ck / 16;
      // S^T tiles: key tile kt holds keys c0 + 16 kt + 4 g + (0..3) of the lane's head column
      f32x4 S[4][NHT], D[4][NHT];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        if (kt < nkt) {
          const int64_t krow = (r0 + c0 + 16 * kt + l16) * a.n2 + kvh;
          uint4 kx[KS];
#pragma unroll
          for (int s = 0; s < KS; ++s) kx[s] = ldg16(k + krow * DQK + 32 * s + 8 * g);
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) acc = Mma<T>::run(as_v8<T>(kx[s]), Qf[ht][s], acc);
            S[kt][ht] = acc * a.scale_log2e;
          }
          if constexpr (DROW) {
            uint4 vx[VS];
#pragma unroll
            for (int s = 0; s < VS; ++s) vx[s] = ldg16(v + krow * DV + 32 * s + 8 * g);
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) {
              f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int s = 0; s < VS; ++s) acc = Mma<T>::run(as_v8<T>(vx[s]), Yf[ht][s], acc);
              D[kt][ht] = acc;
            }
          }
        }
      }
      if constexpr (DROW) {
        // P dP summed over the chunk's keys, per head
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          float acc = 0.f;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            if (kt < nkt) {
#pragma unroll
              for (int e = 0; e < 4; ++e) acc += __builtin_amdgcn_exp2f(S[kt][ht][e] - lse[ht]) * D[kt][ht][e];
            }
          }
          lrun[ht] += acc;
        }
      } else {
        // value rows of the chunk into the LDS tile (rows ck .. up to the next 32 are zero):
        // row 4 j + lane / 16, chunk lane % 16 (16-byte pieces of a 256-byte row)
        constexpr int CPR = DV / 8;  // 16-byte chunks per row
        const int nrow = (ck + 31) / 32 * 32;
        for (int rr = lane / CPR; rr < nrow; rr += 64 / CPR) {
          const int c = lane % CPR;
          uint4 x = make_uint4(0, 0, 0, 0);
          if (rr < ck) x = ldg16(v + ((r0 + c0 + rr) * a.n2 + kvh) * DV + 8 * c);
          lds_st16_at(vt + TV::off(rr, c), x);
        }
        // online softmax: new maximum per head, rescale, P^T in place
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          float mx = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
            if (kt < nkt) mx = fmaxf(mx, max4(S[kt][ht]));
          mx = group_max(mx);
          const float mnew = fmaxf(mrun[ht], mx);
          const float alpha = __builtin_amdgcn_exp2f(mrun[ht] - mnew);  // 0 on the first chunk
          mrun[ht] = mnew;
          float sum = 0.f;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            if (kt < nkt) {
#pragma unroll
              for (int e = 0; e < 4; ++e) S[kt][ht][e] = __builtin_amdgcn_exp2f(S[kt][ht][e] - mnew);
              sum += sum4(S[kt][ht]);
            } else {
              S[kt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
          lrun[ht] = lrun[ht] * alpha + group_sum(sum);
#pragma unroll
          for (int f = 0; f < NF; ++f) O[ht][f] *= alpha;
        }
        asm volatile("" ::: "memory");  // the LDS tile is written before it is read (one wave, in order)
        // O^T += V^T P^T over the chunk: k-step kk covers keys 32 kk .. +31 (tiles 2 kk, 2 kk + 1)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (32 * kk < ck) {
            V8 pb[NHT];
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) pb[ht] = pack8t<T>(S[2 * kk][ht], S[2 * kk + 1][ht]);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
              const uint32_t o = vt + TV::colB(lane, f) + 32 * kk * TV::RB;
              const V8 va = __builtin_bit_cast(V8, join8(lds_tr16_at(o), lds_tr16_at(o + 16 * TV::RB)));
#pragma unroll
              for (int ht = 0; ht < NHT; ++ht) O[ht][f] = Mma<T>::run(va, pb[ht], O[ht][f]);
            }
          }
        }
        asm volatile("" ::: "memory");  // reads of this tile come before the next chunk's writes
      }
    }
  }

  // ---- outputs ----
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = 16 * ht + l16;
    if (h >= G) continue;
    const int64_t row = t * a.n1 + (int64_t)kvh * G + h;
    if constexpr (DROW) {
      const float d = group_sum(lrun[ht]);
      if (g == 0) a.ndrow[row] = -d;
    } else {
      const float l = lrun[ht];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      T* o = static_cast<T*>(a.o) + row * DV;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        // lane holds features 16 f + 4 g .. + 3 of head h
        const uint2 w = make_uint2(pack2<T>(O[ht][f][0] * inv, O[ht][f][1] * inv),
                                   pack2<T>(O[ht][f][2] * inv, O[ht][f][3] * inv));
        *reinterpret_cast<uint2*>(o + 16 * f + 4 * g) = w;
      }
      // statistics in natural units: m = m2 ln 2 (m2 = max s scale log2 e), l as summed
      const float m = l > 0.f ? mrun[ht] * 0.6931471805599453f : -INFINITY;
      const f32x4 val = (g < 2) ? f32x4{m, m, m, m} : f32x4{l, l, l, l};
      float* dst = (g < 2 ? a.smax : a.ssum) + row * 8 + 4 * (g & 1);
      *reinterpret_cast<f32x4*>(dst) = val;
    }
  }
}

template <typename T, bool DROW>
hipError_t launch_t(const SelFwdArgs& a, hipStream_t s) {
  const int64_t units = a.T1 * a.n2;
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)((units + 3) / 4)), block(256);
  const bool two = a.G > 16;
  if (a.d_v != 128) return hipErrorInvalidValue;
  if (a.d_qk == 192) {
    if (two) hipLaunchKernelGGL((sel_fwd_kernel<T, 192, 128, 2, DROW>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((sel_fwd_kernel<T, 192, 128, 1, DROW>), grid, block, 0, s, a);
  } else if (a.d_qk == 128) {
    if (two) hipLaunchKernelGGL((sel_fwd_kernel<T, 128, 128, 2, DROW>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((sel_fwd_kernel<T, 128, 128, 1, DROW>), grid, block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_selected_forward(const SelFwdArgs& a, hipStream_t s) {
  return a.is_f16 ? launch_t<_Float16, false>(a, s) : launch_t<__bf16, false>(a, s);
}

hipError_t launch_selected_drow(const SelFwdArgs& a, hipStream_t s) {
  return a.is_f16 ? launch_t<_Float16, true>(a, s) : launch_t<__bf16, true>(a, s);
}

}  // namespace ab
