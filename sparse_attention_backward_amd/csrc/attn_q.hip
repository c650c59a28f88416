// Query-major dense backward: dQ accumulated in registers (bf16 MFMA, fp32 accumulation).
//
// Page "aclnnFlashAttentionUnpaddingScoreGradV3", Formula section: dQ = dS K / sqrt(d),
// dqRope = dS kRope / sqrt(d), with K = [key, keyRope].
//
// One workgroup (4 waves x 16 query rows) owns a 64-row query tile of one head; the
// rows stay in registers as MFMA B operands and 64-row key tiles pass through LDS (up
// to the diagonal when causal).  Per key tile: S^T = K Q^T and dP^T = V dY^T (A operands
// from LDS), P^T = exp2(S^T*scale*log2e - lse2) and dS^T = P^T (dP^T - drow) -- each lane
// then holds one query row, so lse2 and drow are per-lane scalars -- and dQ += dS K, where
// the dS^T C tiles are the A operand and K is read column-wise with ds_read_b64_tr_b16.
// The next key tile is fetched into registers while the current one is consumed; LDS
// reads run a few MFMAs ahead.  Deterministic: fixed loop order, no atomics.
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

constexpr int kKeys = 64;  // key rows per LDS tile

struct QArgs {
  const uint16_t* q; const uint16_t* q_rope;
  const uint16_t* k; const uint16_t* k_rope;
  const uint16_t* v; const uint16_t* dy;
  const float* lse2; const float* ndrow;
  uint16_t* dq; uint16_t* dq_rope;
  const int64_t* cu_q; const int64_t* cu_kv;
  const int32_t* tiles;  // (sequence, query tile)
  int batch, n1, n2, G, d_main, d_rope, d_v;
  int lo_rel, hi_rel, align;  // mask on j - i (dense_band)
  float scale, scale_log2e;
};

template <int DQK, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void dense_dq_kernel(QArgs a) {
  using SK = Swz<DQK>;
  using SV = Swz<DV>;
  constexpr int KS = DQK / 32, VS = DV / 32, NQ = DQK / 16;
  constexpr int KCH = DQK / 8, VCH = DV / 8;
  constexpr int KPT = KCH / 4, VPT = VCH / 4;  // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kKeys * DQK];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kKeys * DV];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4, jj = l16 >> 2, qq = l16 & 3;
  const int b = a.tiles[2 * blockIdx.x], qt = a.tiles[2 * blockIdx.x + 1];
  const int h = blockIdx.y, kvh = h / a.G;
  const int64_t qs = a.cu_q[b], ks = a.cu_kv[b];
  const int S1 = (int)(a.cu_q[b + 1] - qs), S2 = (int)(a.cu_kv[b + 1] - ks);

  // this lane's query row (B-operand column, and the column of every S^T tile)
  const int rloc = qt * kKeys + 16 * w + l16;
  const bool rvalid = rloc < S1;
  const int64_t qrow = (qs + rloc) * a.n1 + h;
  bf16x8 Qf[KS], Yf[VS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int d = 32 * s + 8 * g;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (rvalid) x = ldg16(d < a.d_main ? a.q + qrow * a.d_main + d : a.q_rope + qrow * a.d_rope + (d - a.d_main));
    Qf[s] = __builtin_bit_cast(bf16x8, x);
  }
#pragma unroll
  for (int s = 0; s < VS; ++s) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (rvalid) x = ldg16(a.dy + qrow * a.d_v + 32 * s + 8 * g);
    Yf[s] = __builtin_bit_cast(bf16x8, x);
  }
  const float lse = rvalid ? a.lse2[qrow] : INFINITY;
  const float ndr = rvalid ? a.ndrow[qrow] : 0.f;

  f32x4 dQ[NQ];
#pragma unroll
  for (int n = 0; n < NQ; ++n) dQ[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // key tiles [klo, khi) hold every key some row of this tile sees: lo <= j - i <= hi
  int lo, hi, klo, khi;
  dense_band(a.lo_rel, a.hi_rel, a.align, S1, S2, lo, hi);
  dense_key_tiles(lo, hi, (int64_t)qt * kKeys, min((qt + 1) * kKeys, S1), S2, kKeys, klo, khi);

  // key-tile loads: thread serves row my_r = tid / 4 and chunks my_c + 4k
  const int my_r = tid >> 2, my_c = tid & 3;
  uint4 pk[KPT], pv[VPT];
  auto prefetch = [&](int kt) {
    const int key = kt * kKeys + my_r;
    const bool ok = key < S2;
    const int64_t kr = (ks + key) * a.n2 + kvh;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int d = 8 * (my_c + 4 * k);
      pk[k] = make_uint4(0, 0, 0, 0);
      if (ok) pk[k] = ldg16(d < a.d_main ? a.k + kr * a.d_main + d : a.k_rope + kr * a.d_rope + (d - a.d_main));
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      pv[k] = make_uint4(0, 0, 0, 0);
      if (ok) pv[k] = ldg16(a.v + kr * a.d_v + 8 * (my_c + 4 * k));
    }
  };

  if (khi > klo) prefetch(klo);
  for (int kt = klo; kt < khi; ++kt) {
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KPT; ++k) sts16(&Ks[SK::off(my_r, 8 * (my_c + 4 * k))], pk[k]);
#pragma unroll
    for (int k = 0; k < VPT; ++k) sts16(&Vs[SV::off(my_r, 8 * (my_c + 4 * k))], pv[k]);
    __syncthreads();
    if (kt + 1 < khi) prefetch(kt + 1);

    // S^T, dP^T: items i = (k-step gi, key sub-tile c); A fragments PD1 items ahead
    constexpr int NI1 = 4 * (KS + VS), PD1 = 4;
    f32x4 ST[4], PT[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) { ST[c] = f32x4{0.f, 0.f, 0.f, 0.f}; PT[c] = ST[c]; }
    auto a1 = [&](int i) -> bf16x8 {
      const int gi = i >> 2, c = i & 3;
      return gi < KS ? lds_read_b128(&Ks[SK::off(16 * c + l16, 32 * gi + 8 * g)])
                     : lds_read_b128(&Vs[SV::off(16 * c + l16, 32 * (gi - KS) + 8 * g)]);
    };
    bf16x8 ring1[PD1];
#pragma unroll
    for (int i = 0; i < PD1; ++i) ring1[i] = a1(i);
#pragma unroll
    for (int i = 0; i < NI1; ++i) {
      const int gi = i >> 2, c = i & 3;
      const bf16x8 x = ring1[i % PD1];
      if (i + PD1 < NI1) ring1[i % PD1] = a1(i + PD1);
      if (gi < KS) ST[c] = mfma_16x16x32(x, Qf[gi], ST[c]);
      else PT[c] = mfma_16x16x32(x, Yf[gi - KS], PT[c]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kt * kKeys + 16 * c + 4 * g + i;
        float p = __builtin_amdgcn_exp2f(ST[c][i] * a.scale_log2e - lse);
        if (key >= S2 || key - rloc < lo || key - rloc > hi) p = 0.f;
        ST[c][i] = p * (PT[c][i] + ndr);
      }
    }
    // dQ += dS K over the two 32-key halves; K column fragments PD2 items ahead
    const bf16x8 da[2] = {pack8(ST[0], ST[1]), pack8(ST[2], ST[3])};
    constexpr int NI2 = 2 * NQ, PD2 = 4;
    auto b2 = [&](int i) -> bf16x8 {
      const int ks2 = i / NQ, nt = i - (i / NQ) * NQ;
      const int r = 32 * ks2 + 4 * g + jj, col = 16 * nt + 4 * qq;
      return join8(lds_read_tr16(&Ks[SK::off(r, col)]), lds_read_tr16(&Ks[SK::off(r + 16, col)]));
    };
    bf16x8 ring2[PD2];
#pragma unroll
    for (int i = 0; i < PD2; ++i) ring2[i] = b2(i);
#pragma unroll
    for (int i = 0; i < NI2; ++i) {
      const int ks2 = i / NQ, nt = i - (i / NQ) * NQ;
      const bf16x8 bk = ring2[i % PD2];
      if (i + PD2 < NI2) ring2[i % PD2] = b2(i + PD2);
      dQ[nt] = mfma_16x16x32(da[ks2], bk, dQ[nt]);
    }
  }

  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < NQ; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) Ks[SK::off(16 * w + 4 * g + i, 16 * nt + l16)] = f2bf(dQ[nt][i] * a.scale);
  __syncthreads();
  for (int idx = tid; idx < kKeys * KCH; idx += 256) {
    const int r = idx / KCH, d = 8 * (idx - r * KCH);
    const int rl = qt * kKeys + r;
    if (rl < S1) {
      const int64_t qr = (qs + rl) * a.n1 + h;
      uint16_t* dst = d < a.d_main ? a.dq + qr * a.d_main + d : a.dq_rope + qr * a.d_rope + (d - a.d_main);
      sts16(dst, *reinterpret_cast<const uint4*>(&Ks[SK::off(r, d)]));
    }
  }
}

}  // namespace

hipError_t launch_dense_dq_bf16(const DenseArgs& a, hipStream_t s) {
  if (a.n_q_tiles == 0) return hipSuccess;
  QArgs k{};
  k.q = (const uint16_t*)a.q; k.q_rope = (const uint16_t*)a.q_rope;
  k.k = (const uint16_t*)a.k; k.k_rope = (const uint16_t*)a.k_rope;
  k.v = (const uint16_t*)a.v; k.dy = (const uint16_t*)a.dy;
  k.lse2 = a.lse2; k.ndrow = a.ndrow;
  k.dq = (uint16_t*)a.dq; k.dq_rope = (uint16_t*)a.dq_rope;
  k.cu_q = a.cu_q; k.cu_kv = a.cu_kv; k.tiles = a.q_tiles;
  k.batch = a.batch; k.n1 = a.n1; k.n2 = a.n2; k.G = a.G;
  k.d_main = a.d_main; k.d_rope = a.d_rope; k.d_v = a.d_v;
  k.lo_rel = a.mask_on ? a.lo_rel : -kBandInf; k.hi_rel = a.mask_on ? a.hi_rel : kBandInf; k.align = a.align;
  k.scale = a.scale; k.scale_log2e = a.scale_log2e;
  const dim3 grid(a.n_q_tiles, a.n1);
  const int dqk = a.d_main + a.d_rope;
  if (dqk == 192 && a.d_v == 128) hipLaunchKernelGGL((dense_dq_kernel<192, 128>), grid, dim3(256), 0, s, k);
  else if (dqk == 128 && a.d_v == 128) hipLaunchKernelGGL((dense_dq_kernel<128, 128>), grid, dim3(256), 0, s, k);
  else if (dqk == 64 && a.d_v == 64) hipLaunchKernelGGL((dense_dq_kernel<64, 64>), grid, dim3(256), 0, s, k);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ab
