// Dense varlen backward in fp32 on the vector ALUs (no MFMA): the precision path.
//
// Page "aclnnFlashAttentionUnpaddingScoreGradV3", Formula section; the same math as
// the bf16 MFMA kernels, with fp32 operands and fp32 fused multiply-adds throughout:
//   dense_kv_fp32: one workgroup per (key row j, KV head): for every query row (i, h)
//     of the head's group that sees j, p = exp2(q.k * scale*log2e - lse2),
//     dp = dY.v, ds = p (dp - drow); dV_j += p dY_i, dK_j += ds Q_i; dK_j *= scale.
//   dense_dq_fp32: one workgroup per (query row i, head h): dQ_i = scale * sum_j ds_j K_j.
// Both are deterministic (fixed loop order, no atomics).
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

constexpr int kF32MaxD = 256;  // max head dim (qk incl. rope, and v) of this path

__device__ __forceinline__ float qk_elem(const float* main, const float* rope, int64_t row, int nh, int h,
                                         int d_main, int d_rope, int d) {
  return d < d_main ? main[(row * nh + h) * d_main + d] : rope[(row * nh + h) * d_rope + (d - d_main)];
}

__global__ __launch_bounds__(64) void dense_kv_fp32(DenseArgs a) {
  __shared__ float Kj[kF32MaxD], Vj[kF32MaxD], p_s[64], ds_s[64];
  const int tid = threadIdx.x;
  const int64_t j = blockIdx.x;
  const int kvh = blockIdx.y;
  const int dqk = a.d_main + a.d_rope, dv = a.d_v;
  const float* q = (const float*)a.q; const float* qr = (const float*)a.q_rope;
  const float* k = (const float*)a.k; const float* kr = (const float*)a.k_rope;
  const float* v = (const float*)a.v; const float* dy = (const float*)a.dy;
  const int b = seq_of(a.cu_kv, a.batch, j);
  const int64_t jloc = j - a.cu_kv[b];
  const int64_t qs = a.cu_q[b], qe = a.cu_q[b + 1];
  for (int d = tid; d < dqk; d += 64) Kj[d] = qk_elem(k, kr, j, a.n2, kvh, a.d_main, a.d_rope, d);
  for (int d = tid; d < dv; d += 64) Vj[d] = v[(j * a.n2 + kvh) * dv + d];
  __syncthreads();
  float dk[kF32MaxD / 64], dvv[kF32MaxD / 64];
#pragma unroll
  for (int c = 0; c < kF32MaxD / 64; ++c) dk[c] = dvv[c] = 0.f;
  // query rows that see key j: lo <= j - i <= hi
  int lo, hi;
  dense_band(a.lo_rel, a.hi_rel, a.align, qe - qs, a.cu_kv[b + 1] - a.cu_kv[b], lo, hi);
  const int64_t ia = jloc - hi > 0 ? jloc - hi : 0, ib = jloc - lo < qe - qs ? jloc - lo + 1 : qe - qs;
  const int64_t i0 = qs + ia;
  const int64_t R = (ib > ia ? ib - ia : 0) * a.G;
  for (int64_t r0 = 0; r0 < R; r0 += 64) {
    float p = 0.f, ds = 0.f;
    const int64_t r = r0 + tid;
    if (r < R) {
      const int64_t i = i0 + r / a.G;
      const int h = kvh * a.G + (int)(r % a.G);
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < dqk; ++d) s = fmaf(qk_elem(q, qr, i, a.n1, h, a.d_main, a.d_rope, d), Kj[d], s);
      for (int d = 0; d < dv; ++d) dp = fmaf(dy[(i * a.n1 + h) * dv + d], Vj[d], dp);
      p = exp2f(s * a.scale_log2e - a.lse2[i * a.n1 + h]);
      ds = p * (dp + a.ndrow[i * a.n1 + h]);
    }
    p_s[tid] = p;
    ds_s[tid] = ds;
    __syncthreads();
    const int nr = (int)((R - r0) < 64 ? (R - r0) : 64);
    for (int rr = 0; rr < nr; ++rr) {
      const int64_t i = i0 + (r0 + rr) / a.G;
      const int h = kvh * a.G + (int)((r0 + rr) % a.G);
#pragma unroll
      for (int c = 0; c < kF32MaxD / 64; ++c) {
        const int d = tid + 64 * c;
        if (d < dqk) dk[c] = fmaf(ds_s[rr], qk_elem(q, qr, i, a.n1, h, a.d_main, a.d_rope, d), dk[c]);
        if (d < dv) dvv[c] = fmaf(p_s[rr], dy[(i * a.n1 + h) * dv + d], dvv[c]);
      }
    }
    __syncthreads();
  }
  float* dko = (float*)a.dk; float* dkr = (float*)a.dk_rope; float* dvo = (float*)a.dv;
#pragma unroll
  for (int c = 0; c < kF32MaxD / 64; ++c) {
    const int d = tid + 64 * c;
    if (d < a.d_main) dko[(j * a.n2 + kvh) * a.d_main + d] = dk[c] * a.scale;
    else if (d < dqk) dkr[(j * a.n2 + kvh) * a.d_rope + (d - a.d_main)] = dk[c] * a.scale;
    if (d < dv) dvo[(j * a.n2 + kvh) * dv + d] = dvv[c];
  }
}

__global__ __launch_bounds__(64) void dense_dq_fp32(DenseArgs a) {
  __shared__ float Qi[kF32MaxD], Yi[kF32MaxD], ds_s[64];
  const int tid = threadIdx.x;
  const int64_t i = blockIdx.x;
  const int h = blockIdx.y;
  const int kvh = h / a.G;
  const int dqk = a.d_main + a.d_rope, dv = a.d_v;
  const float* q = (const float*)a.q; const float* qr = (const float*)a.q_rope;
  const float* k = (const float*)a.k; const float* kr = (const float*)a.k_rope;
  const float* v = (const float*)a.v; const float* dy = (const float*)a.dy;
  const int b = seq_of(a.cu_q, a.batch, i);
  const int64_t iloc = i - a.cu_q[b];
  const int64_t ks = a.cu_kv[b], ke = a.cu_kv[b + 1];
  // keys that query i sees: lo <= j - i <= hi
  int lo, hi;
  dense_band(a.lo_rel, a.hi_rel, a.align, a.cu_q[b + 1] - a.cu_q[b], ke - ks, lo, hi);
  const int64_t kbeg = iloc + lo > 0 ? ks + iloc + lo : ks;
  const int64_t kend = iloc + hi < ke - ks ? ks + iloc + hi + 1 : ke;
  for (int d = tid; d < dqk; d += 64) Qi[d] = qk_elem(q, qr, i, a.n1, h, a.d_main, a.d_rope, d);
  for (int d = tid; d < dv; d += 64) Yi[d] = dy[(i * a.n1 + h) * dv + d];
  const float lse2 = a.lse2[i * a.n1 + h], ndrow = a.ndrow[i * a.n1 + h];
  __syncthreads();
  float acc[kF32MaxD / 64];
#pragma unroll
  for (int c = 0; c < kF32MaxD / 64; ++c) acc[c] = 0.f;
  for (int64_t j0 = kbeg; j0 < kend; j0 += 64) {
    const int64_t j = j0 + tid;
    float ds = 0.f;
    if (j < kend) {
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < dqk; ++d) s = fmaf(Qi[d], qk_elem(k, kr, j, a.n2, kvh, a.d_main, a.d_rope, d), s);
      for (int d = 0; d < dv; ++d) dp = fmaf(Yi[d], v[(j * a.n2 + kvh) * dv + d], dp);
      const float p = exp2f(s * a.scale_log2e - lse2);
      ds = p * (dp + ndrow);
    }
    ds_s[tid] = ds;
    __syncthreads();
    const int nj = (int)((kend - j0) < 64 ? (kend - j0) : 64);
    for (int jj = 0; jj < nj; ++jj) {
#pragma unroll
      for (int c = 0; c < kF32MaxD / 64; ++c) {
        const int d = tid + 64 * c;
        if (d < dqk) acc[c] = fmaf(ds_s[jj], qk_elem(k, kr, j0 + jj, a.n2, kvh, a.d_main, a.d_rope, d), acc[c]);
      }
    }
    __syncthreads();
  }
  float* dqo = (float*)a.dq; float* dqr = (float*)a.dq_rope;
#pragma unroll
  for (int c = 0; c < kF32MaxD / 64; ++c) {
    const int d = tid + 64 * c;
    if (d < a.d_main) dqo[(i * a.n1 + h) * a.d_main + d] = acc[c] * a.scale;
    else if (d < dqk) dqr[(i * a.n1 + h) * a.d_rope + (d - a.d_main)] = acc[c] * a.scale;
  }
}

hipError_t launch_dense_fp32(const DenseArgs& a, hipStream_t s) {
  if (a.T2 > 0) hipLaunchKernelGGL(dense_kv_fp32, dim3((unsigned)a.T2, a.n2), dim3(64), 0, s, a);
  if (a.T1 > 0) hipLaunchKernelGGL(dense_dq_fp32, dim3((unsigned)a.T1, a.n1), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace ab
