// Row statistics for the backward pass (both forms); the same launch also copies the call's
// tables (schedule, sequence offsets) from pinned host memory into the workspace.
//
// For every query row (t, h):
//   lse2 = (softmaxMax + ln softmaxSum) * log2(e), so that P = exp2(s * scale * log2(e) - lse2)
//          reproduces exp(s * scale - m) / l; a row with l = 0 (no visible key) gets +inf,
//          which makes every P of that row 0.
//   ndrow = -sum_d dY[t,h,d] * O[t,h,d], minus rowsum(P * dP) because O = P V; stored negated
//          so that a dP accumulator started at ndrow ends at dP - rowsum(P * dP).  Not written
//          when O is not given (the selected form then forms it from P and dP).
// softmaxMax / softmaxSum are [T, N, 8] float32 with identical lanes; lane 0 is read.
// HBM-bound: 2 * d_v * sizeof(T) + 64 bytes moved per row (the stats rows are 32 B
// each but a 4-byte read of each touches one 32-byte sector).
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

__device__ __forceinline__ float dot16(uint4 a, uint4 b, uint16_t) {
  float s = 0.f;
  const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += __uint_as_float(av[i] << 16) * __uint_as_float(bv[i] << 16);
    s += __uint_as_float(av[i] & 0xffff0000u) * __uint_as_float(bv[i] & 0xffff0000u);
  }
  return s;
}

__device__ __forceinline__ float dot16(uint4 a, uint4 b, _Float16) {
  float s = 0.f;
  const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += t2f<_Float16>((uint16_t)(av[i] & 0xffffu)) * t2f<_Float16>((uint16_t)(bv[i] & 0xffffu));
    s += t2f<_Float16>((uint16_t)(av[i] >> 16)) * t2f<_Float16>((uint16_t)(bv[i] >> 16));
  }
  return s;
}

__device__ __forceinline__ float dot16(uint4 a, uint4 b, float) {
  return __uint_as_float(a.x) * __uint_as_float(b.x) + __uint_as_float(a.y) * __uint_as_float(b.y) +
         __uint_as_float(a.z) * __uint_as_float(b.z) + __uint_as_float(a.w) * __uint_as_float(b.w);
}

// LPR lanes cooperate on one row; each lane reads 16-byte chunks.  A wave takes kRowU
// groups of 64 / LPR rows per pass, their loads issued together (more bytes in flight per
// wave, fewer workgroups to dispatch).
constexpr int kRowU = 4;
template <typename T, int LPR>
__global__ __launch_bounds__(256) void preprocess_kernel(PreArgs a) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR;
  // the call's tables: pinned host memory -> workspace (read by the kernels that follow)
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, nthreads = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = gtid; i < a.tab_n16; i += nthreads) a.tab_dst[i] = a.tab_src[i];
  const int64_t wave = gtid >> 6;
  const int64_t nwaves = nthreads >> 6;
  for (int64_t base = wave * RPW * kRowU; base < a.rows; base += nwaves * RPW * kRowU) {
    float acc[kRowU];
#pragma unroll
    for (int u = 0; u < kRowU; ++u) {
      const int64_t row = base + u * RPW + lane / LPR;
      acc[u] = 0.f;
      if (row < a.rows && a.out) {
        const T* o = reinterpret_cast<const T*>(a.out) + row * a.dv;
        const T* d = reinterpret_cast<const T*>(a.dy) + row * a.dv;
        for (int c = sub * VEC; c < a.dv; c += LPR * VEC) acc[u] += dot16(ldg16(o + c), ldg16(d + c), T());
      }
    }
#pragma unroll
    for (int u = 0; u < kRowU; ++u) {
      const int64_t row = base + u * RPW + lane / LPR;
      float s = acc[u];
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
      if (sub == 0 && row < a.rows) {
        if (a.out) a.ndrow[row] = -s;  // without O the row statistic comes from another pass
        const float m = a.smax[row * 8], l = a.ssum[row * 8];
        a.lse2[row] = (l > 0.f && m > -INFINITY) ? (m + logf(l)) * kLog2e : INFINITY;
      }
    }
  }
}

template <typename T>
static hipError_t launch_pre_t(const PreArgs& a, hipStream_t s) {
  constexpr int VEC = 16 / sizeof(T);
  int chunks = a.dv / VEC, lpr = 1;
  while (lpr * 2 <= chunks && lpr < 64) lpr *= 2;
  const int64_t rows_per_block = 4 * (64 / lpr) * kRowU;
  int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 2048) blocks = 2048;  // about what the device holds at once; the rest loop
  if (blocks < 1) blocks = 1;
  dim3 grid((unsigned)blocks), block(256);
  switch (lpr) {
    case 1: hipLaunchKernelGGL((preprocess_kernel<T, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((preprocess_kernel<T, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((preprocess_kernel<T, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((preprocess_kernel<T, 8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((preprocess_kernel<T, 16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((preprocess_kernel<T, 32>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((preprocess_kernel<T, 64>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_preprocess(const PreArgs& a, hipStream_t s) {
  if (a.rows == 0 && a.tab_n16 == 0) return hipSuccess;
  if (a.elem == 1) return launch_pre_t<_Float16>(a, s);
  return a.elem == 2 ? launch_pre_t<float>(a, s) : launch_pre_t<uint16_t>(a, s);
}

}  // namespace ab
