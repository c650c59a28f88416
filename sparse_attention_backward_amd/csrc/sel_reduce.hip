// dQ of the selected form from the per-block partials left by the KV-major kernel.
//
// Page "NsaSelectedAttentionGrad", formula section: dQ = dS K / sqrt(d) over the gathered
// rows, i.e. the sum over the selected blocks of each block's dS_block K_block.  The
// KV-major kernel stores every block's share (bf16, G x DQK) at [t - t0, slot, kvh] for the
// tokens [t0, t1) of the current window (the list entry t cnt + slot, less t0 cnt, times n2,
// plus kvh: no division in the store address), its 16-byte chunks permuted as share_chunk
// says; this kernel adds the slots of each (token, KV head) of the window chunk by chunk in
// slot order, scales, and writes each chunk to its place (share_pos):
//   dQ[t, kvh G + h, :] = scale * sum_slot part[t, slot, kvh](h, :).
// Fixed order, one writer per output row: deterministic.
//
// One wave per (token, KV head).  Lane l owns the 16-byte chunks l, l + 64, ... of the
// G x DQK block (six per lane at G = 16, DQK = 192), and the slot loop takes two slots per
// iteration so that twelve 16-byte loads per lane are in flight.  A slot whose topk id is
// out of range was never written and is skipped: the ids are checked once, one ballot per
// 64 slots.  Shares and dQ are touched once: streaming (non-temporal) loads and stores.
#include "common.hpp"
#include "kernels.hpp"
#include "share_layout.hpp"

namespace ab {

namespace {

constexpr int kU = 6;  // chunks per lane per pass
constexpr uint32_t kNegZero2 = 0x80008000u;  // two -0.0 (bf16 and fp16 alike): x + (-0) == x for every x

template <typename T>
__device__ __forceinline__ void add_x8(float* acc, const uint4& x) {
  const uint32_t xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc[2 * j] += t2f<T>((uint16_t)(xv[j] & 0xffffu));
    acc[2 * j + 1] += t2f<T>((uint16_t)(xv[j] >> 16));
  }
}

template <typename T, int DQK>
__global__ __launch_bounds__(256) void dq_reduce_kernel(const uint16_t* part, uint16_t* dq, int64_t t0, int64_t pairs,
                                                        int n2, int n1, int G, int cnt, float scale,
                                                        const int32_t* topk, const int64_t* cu_q,
                                                        const int32_t* blkoff, int batch) {
  const int lane = threadIdx.x & 63;
  const int64_t wpair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // within the window
  if (wpair >= pairs) return;  // whole wave
  const int64_t tw = wpair / n2, t = t0 + tw, pair = t0 * n2 + wpair;
  const int kvh = (int)(wpair - tw * n2);
  const int b = seq_of(cu_q, batch, t);
  const int nblk = blkoff[b + 1] - blkoff[b];
  uint64_t valid[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int sl = 64 * h + lane;
    bool ok = false;
    if (sl < cnt) {
      const int id = topk[pair * cnt + sl];
      ok = id >= 0 && id < nblk;
    }
    valid[h] = __ballot(ok);
  }
  auto slot_ok = [&](int sl) -> bool { return (valid[sl >> 6] >> (sl & 63)) & 1; };
  const int chunks = G * DQK / 8;
  const int R = share_rows(G);
  const int64_t slot_stride = (int64_t)n2 * G * DQK;
  const uint16_t* src = part + (tw * cnt * n2 + kvh) * (int64_t)G * DQK;
  uint16_t* out = dq + (t * n1 + (int64_t)kvh * G) * DQK;
  for (int c0 = lane; c0 < chunks; c0 += 64 * kU) {
    float acc[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[u][j] = 0.f;
    for (int sl = 0; sl < cnt; sl += 2) {
      const bool v0 = slot_ok(sl), v1 = sl + 1 < cnt && slot_ok(sl + 1);
      uint4 x0[kU], x1[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = c0 + 64 * u;
        x0[u] = make_uint4(kNegZero2, kNegZero2, kNegZero2, kNegZero2);  // adds nothing, exactly
        x1[u] = make_uint4(kNegZero2, kNegZero2, kNegZero2, kNegZero2);
        if (v0 && c < chunks) x0[u] = ldg16_stream(src + sl * slot_stride + 8 * c);
        if (v1 && c < chunks) x1[u] = ldg16_stream(src + (sl + 1) * slot_stride + 8 * c);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) add_x8<T>(acc[u], x0[u]);
#pragma unroll
      for (int u = 0; u < kU; ++u) add_x8<T>(acc[u], x1[u]);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + 64 * u;
      if (c < chunks) {
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = (uint32_t)f2t<T>(acc[u][2 * j] * scale) | ((uint32_t)f2t<T>(acc[u][2 * j + 1] * scale) << 16);
        sts16_stream(out + 8 * share_pos<DQK>(c, R), make_uint4(o[0], o[1], o[2], o[3]));
      }
    }
  }
}

}  // namespace

hipError_t launch_selected_dq_reduce(const SelArgs& a, hipStream_t s) {
  const int64_t pairs = (a.t1 - a.t0) * a.n2;  // (token, KV head) pairs of the window
  if (pairs == 0) return hipSuccess;
  const dim3 grid((unsigned)((pairs + 3) / 4)), block(256);
  const uint16_t* part = (const uint16_t*)a.dq_part;
  uint16_t* dq = (uint16_t*)a.dq;
#define AB_DQ_REDUCE(T, D)                                                                                   \
  hipLaunchKernelGGL((dq_reduce_kernel<T, D>), grid, block, 0, s, part, dq, a.t0, pairs, a.n2, a.n1, a.G, a.cnt, \
                     a.scale, a.topk, a.cu_q, a.blkoff, a.batch)
  if (a.d_qk == 192) {
    if (a.is_f16) AB_DQ_REDUCE(_Float16, 192);
    else AB_DQ_REDUCE(__bf16, 192);
  } else if (a.d_qk == 128) {
    if (a.is_f16) AB_DQ_REDUCE(_Float16, 128);
    else AB_DQ_REDUCE(__bf16, 128);
  } else {
    return hipErrorInvalidValue;
  }
#undef AB_DQ_REDUCE
  return hipGetLastError();
}

}  // namespace ab
