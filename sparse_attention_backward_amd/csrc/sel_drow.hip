// Selected (NSA) attention: the row statistic of the backward without attentionOut.
//
// Page "NsaSelectedAttentionGrad", parameter table: attentionOut is optional.  Without it
// the backward's rowsum(dY * O) is formed from its other definition over the gathered rows:
//   drow = sum_j P_j dP_j,  P_j = exp(s_j - m) / l from the passed statistics (lse2),
//   dP = dY V^T,  s = scale Q K^T over the selectedBlockCount blocks that topkIndices
//   gathers for the token and KV head; stored negated (ndrow) for the backward.
//
// One wave per (token, KV head); the four waves of a workgroup are independent.  The G
// query heads are the columns of the MFMA tiles (one 16-column tile for G <= 16, two for
// G <= 32), so every product is computed transposed, with the key rows read from global
// memory 16 bytes per lane as the A operand:
//   S^T (keys x heads)  = K x Q^T (B: the head rows, resident),
//   dP^T (keys x heads) = V x dY^T (B, resident).
// The lane that holds column h of a C tile holds head h: the sum of a head is reduced over
// the lane's 4 values and across its 4 lane groups.  An out-of-range id is skipped (the
// index build of the same call raises the flag).
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

constexpr int kChunk = 64;  // keys per step

template <typename T, int DQK, int DV, int NHT>
__global__ __launch_bounds__(256) void sel_drow_kernel(SelFwdArgs a) {
  using V8 = typename Mma<T>::v8;
  constexpr int KS = DQK / 32, VS = DV / 32;

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
  const T* dy = static_cast<const T*>(a.dy);

  // Q^T and dY^T as B operands: lane column = head 16 ht + l16, k = features 32 s + 8 g ..
  V8 Qf[NHT][KS], Yf[NHT][VS];
  float lse[NHT], acc[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = 16 * ht + l16;
    const int64_t row = t * a.n1 + (int64_t)kvh * G + h;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      Qf[ht][s] = as_v8<T>(h < G ? ldg16(q + row * DQK + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0));
#pragma unroll
    for (int s = 0; s < VS; ++s)
      Yf[ht][s] = as_v8<T>(h < G ? ldg16(dy + row * DV + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0));
    lse[ht] = h < G ? a.lse2[row] : INFINITY;
    acc[ht] = 0.f;
  }
  const int32_t* ids = a.topk + unit * a.cnt;

  for (int i = 0; i < a.cnt; ++i) {
    const int id = __builtin_amdgcn_readfirstlane(ids[i]);
    if (id < 0 || id >= nblk) continue;
    const int64_t r0 = kv0 + (int64_t)id * a.bs;
    for (int c0 = 0; c0 < a.bs; c0 += kChunk) {
      const int nkt = min(kChunk, a.bs - c0) / 16;  // bs is a multiple of 16
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        if (kt < nkt) {
          // key tile kt: keys c0 + 16 kt + 4 g + (0..3) of the lane's head column
          const int64_t krow = (r0 + c0 + 16 * kt + l16) * a.n2 + kvh;
          uint4 kx[KS], vx[VS];
#pragma unroll
          for (int s = 0; s < KS; ++s) kx[s] = ldg16(k + krow * DQK + 32 * s + 8 * g);
#pragma unroll
          for (int s = 0; s < VS; ++s) vx[s] = ldg16(v + krow * DV + 32 * s + 8 * g);
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht) {
            f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, da = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) sa = Mma<T>::run(as_v8<T>(kx[s]), Qf[ht][s], sa);
#pragma unroll
            for (int s = 0; s < VS; ++s) da = Mma<T>::run(as_v8<T>(vx[s]), Yf[ht][s], da);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[ht] += __builtin_amdgcn_exp2f(sa[e] * a.scale_log2e - lse[ht]) * da[e];
          }
        }
      }
    }
  }
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = 16 * ht + l16;
    const float d = group_sum(acc[ht]);
    if (h < G && g == 0) a.ndrow[t * a.n1 + (int64_t)kvh * G + h] = -d;
  }
}

template <typename T>
hipError_t launch_t(const SelFwdArgs& a, hipStream_t s) {
  const int64_t units = a.T1 * a.n2;
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)((units + 3) / 4)), block(256);
  const bool two = a.G > 16;
  if (a.d_v != 128) return hipErrorInvalidValue;
  if (a.d_qk == 192) {
    if (two) hipLaunchKernelGGL((sel_drow_kernel<T, 192, 128, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((sel_drow_kernel<T, 192, 128, 1>), grid, block, 0, s, a);
  } else if (a.d_qk == 128) {
    if (two) hipLaunchKernelGGL((sel_drow_kernel<T, 128, 128, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((sel_drow_kernel<T, 128, 128, 1>), grid, block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_selected_drow(const SelFwdArgs& a, hipStream_t s) {
  return a.is_f16 ? launch_t<_Float16>(a, s) : launch_t<__bf16>(a, s);
}

}  // namespace ab
