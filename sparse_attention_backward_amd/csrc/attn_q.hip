// Query-major backward: dQ accumulated in registers (bf16 MFMA, fp32 accumulation).
//
// Page "aclnnFlashAttentionUnpaddingScoreGradV3", Formula section (dQ = dS K / sqrt(d),
// dqRope = dS kRope / sqrt(d)) and page "NsaSelectedAttentionGrad", formula section
// (dQ over the gathered selectedKey rows).
//
// The query rows of a workgroup stay in registers as MFMA B operands; key tiles of 64
// rows pass through LDS.  Per key tile the kernel computes S^T = K Q^T and
// dP^T = V dY^T (A operands from LDS), P^T = exp2(S^T*scale*log2e - lse2) and
// dS^T = P^T (dP^T - drow) -- each lane then holds one query row, so lse2 and drow are
// per-lane scalars -- and dQ += dS K, where the dS^T C tiles are the A operand and K is
// read column-wise from LDS with ds_read_b64_tr_b16.
//   dense:    4 waves x 16 query rows = one 64-row query tile of one head; key tiles up
//             to the diagonal when causal.
//   selected: one token and KV head; the 16 rows are the G (<= 16) query heads; the
//             cnt*block_size gathered key rows are cut into 64-row tiles and each wave
//             takes 16 of them (16x16x16 MFMA for dQ), wave partials summed at the end.
// Deterministic: fixed loop order, no atomics.
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

constexpr int kKeys = 64;  // key rows per LDS tile
constexpr int kPad = 8;

struct QArgs {
  const uint16_t* q; const uint16_t* q_rope;
  const uint16_t* k; const uint16_t* k_rope;
  const uint16_t* v; const uint16_t* dy;
  const float* lse2; const float* drow;
  uint16_t* dq; uint16_t* dq_rope;
  const int64_t* cu_q; const int64_t* cu_kv;
  const int32_t* tiles;  // dense: (sequence, query tile)
  const int32_t* topk;   // selected
  int batch, n1, n2, G, d_main, d_rope, d_v;
  int causal, bs, cnt;
  float scale, scale_log2e;
};

template <int DQK, int DV>
__global__ __launch_bounds__(256) void dense_dq_kernel(QArgs a) {
  constexpr int KST = DQK + kPad, VST = DV + kPad;
  constexpr int KS = DQK / 32, VS = DV / 32, NQ = DQK / 16;
  constexpr int KCH = DQK / 8, VCH = DV / 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kKeys * KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kKeys * VST];

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
  const float dr = rvalid ? a.drow[qrow] : 0.f;

  f32x4 dQ[NQ];
#pragma unroll
  for (int n = 0; n < NQ; ++n) dQ[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  int nkt = a.causal ? qt + 1 : (S2 + kKeys - 1) / kKeys;
  const int nkt_all = (S2 + kKeys - 1) / kKeys;
  if (nkt > nkt_all) nkt = nkt_all;
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    for (int idx = tid; idx < kKeys * KCH; idx += 256) {
      const int r = idx / KCH, d = 8 * (idx - r * KCH);
      const int key = kt * kKeys + r;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (key < S2) {
        const int64_t kr = (ks + key) * a.n2 + kvh;
        x = ldg16(d < a.d_main ? a.k + kr * a.d_main + d : a.k_rope + kr * a.d_rope + (d - a.d_main));
      }
      sts16(&Ks[r * KST + d], x);
    }
    for (int idx = tid; idx < kKeys * VCH; idx += 256) {
      const int r = idx / VCH, d = 8 * (idx - r * VCH);
      const int key = kt * kKeys + r;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (key < S2) x = ldg16(a.v + ((ks + key) * a.n2 + kvh) * a.d_v + d);
      sts16(&Vs[r * VST + d], x);
    }
    __syncthreads();

    f32x4 ST[4], PT[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ST[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      PT[c] = ST[c];
#pragma unroll
      for (int s = 0; s < KS; ++s) ST[c] = mfma_16x16x32(lds_read_b128(&Ks[(16 * c + l16) * KST + 32 * s + 8 * g]), Qf[s], ST[c]);
#pragma unroll
      for (int s = 0; s < VS; ++s) PT[c] = mfma_16x16x32(lds_read_b128(&Vs[(16 * c + l16) * VST + 32 * s + 8 * g]), Yf[s], PT[c]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kt * kKeys + 16 * c + 4 * g + i;
        float p = __builtin_amdgcn_exp2f(ST[c][i] * a.scale_log2e - lse);
        if (key >= S2 || (a.causal && key > rloc)) p = 0.f;
        ST[c][i] = p * (PT[c][i] - dr);
      }
    }
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const bf16x8 da = pack8(ST[2 * ks2], ST[2 * ks2 + 1]);
#pragma unroll
      for (int nt = 0; nt < NQ; ++nt) {
        const uint16_t* p = &Ks[(32 * ks2 + 4 * g + jj) * KST + 16 * nt + 4 * qq];
        dQ[nt] = mfma_16x16x32(da, join8(lds_read_tr16(p), lds_read_tr16(p + 16 * KST)), dQ[nt]);
      }
    }
  }

  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < NQ; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) Ks[(16 * w + 4 * g + i) * KST + 16 * nt + l16] = f2bf(dQ[nt][i] * a.scale);
  __syncthreads();
  for (int idx = tid; idx < kKeys * KCH; idx += 256) {
    const int r = idx / KCH, d = 8 * (idx - r * KCH);
    const int rl = qt * kKeys + r;
    if (rl < S1) {
      const int64_t qr = (qs + rl) * a.n1 + h;
      uint16_t* dst = d < a.d_main ? a.dq + qr * a.d_main + d : a.dq_rope + qr * a.d_rope + (d - a.d_main);
      sts16(dst, *reinterpret_cast<const uint4*>(&Ks[r * KST + d]));
    }
  }
}

template <int DQK, int DV>
__global__ __launch_bounds__(256) void sel_dq_kernel(QArgs a) {
  constexpr int KST = DQK + kPad, VST = DV + kPad;
  constexpr int KS = DQK / 32, VS = DV / 32, NQ = DQK / 16;
  constexpr int KCH = DQK / 8, VCH = DV / 8;
  constexpr int SMEM = kKeys * KST + kKeys * VST;
  static_assert(SMEM * 2 >= 3 * 16 * DQK * 4, "reduction buffer must fit in the staging area");
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM];
  __shared__ int ids_s[128];
  uint16_t* Ks = smem;
  uint16_t* Vs = smem + kKeys * KST;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4, jj = l16 >> 2, qq = l16 & 3;
  const int64_t u = blockIdx.x;
  const int64_t t = u / a.n2;
  const int kvh = (int)(u - t * a.n2);
  const int b = seq_of(a.cu_q, a.batch, t);
  const int64_t kv0 = a.cu_kv[b];
  const int nblk = (int)((a.cu_kv[b + 1] - kv0) / a.bs);
  if (tid < a.cnt) {
    const int id = a.topk[(t * a.n2 + kvh) * a.cnt + tid];
    ids_s[tid] = (id >= 0 && id < nblk) ? id : -1;  // out-of-range ids contribute nothing
  }

  const bool rvalid = l16 < a.G;
  const int64_t qrow = t * a.n1 + kvh * a.G + l16;
  bf16x8 Qf[KS], Yf[VS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (rvalid) x = ldg16(a.q + qrow * DQK + 32 * s + 8 * g);
    Qf[s] = __builtin_bit_cast(bf16x8, x);
  }
#pragma unroll
  for (int s = 0; s < VS; ++s) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (rvalid) x = ldg16(a.dy + qrow * DV + 32 * s + 8 * g);
    Yf[s] = __builtin_bit_cast(bf16x8, x);
  }
  const float lse = rvalid ? a.lse2[qrow] : INFINITY;
  const float dr = rvalid ? a.drow[qrow] : 0.f;

  f32x4 dQ[NQ];
#pragma unroll
  for (int n = 0; n < NQ; ++n) dQ[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsel = a.cnt * a.bs;
  const int ntiles = (nsel + kKeys - 1) / kKeys;
  for (int tile = 0; tile < ntiles; ++tile) {
    __syncthreads();  // ids_s ready / previous tile consumed
    for (int idx = tid; idx < kKeys * KCH; idx += 256) {
      const int r = idx / KCH, d = 8 * (idx - r * KCH);
      const int kk = tile * kKeys + r;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (kk < nsel) {
        const int slot = kk / a.bs, id = ids_s[slot];
        if (id >= 0) x = ldg16(a.k + ((kv0 + (int64_t)id * a.bs + (kk - slot * a.bs)) * a.n2 + kvh) * DQK + d);
      }
      sts16(&Ks[r * KST + d], x);
    }
    for (int idx = tid; idx < kKeys * VCH; idx += 256) {
      const int r = idx / VCH, d = 8 * (idx - r * VCH);
      const int kk = tile * kKeys + r;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (kk < nsel) {
        const int slot = kk / a.bs, id = ids_s[slot];
        if (id >= 0) x = ldg16(a.v + ((kv0 + (int64_t)id * a.bs + (kk - slot * a.bs)) * a.n2 + kvh) * DV + d);
      }
      sts16(&Vs[r * VST + d], x);
    }
    __syncthreads();

    f32x4 ST = f32x4{0.f, 0.f, 0.f, 0.f}, PT = ST;
#pragma unroll
    for (int s = 0; s < KS; ++s) ST = mfma_16x16x32(lds_read_b128(&Ks[(16 * w + l16) * KST + 32 * s + 8 * g]), Qf[s], ST);
#pragma unroll
    for (int s = 0; s < VS; ++s) PT = mfma_16x16x32(lds_read_b128(&Vs[(16 * w + l16) * VST + 32 * s + 8 * g]), Yf[s], PT);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = tile * kKeys + 16 * w + 4 * g + i;
      float p = __builtin_amdgcn_exp2f(ST[i] * a.scale_log2e - lse);
      if (kk >= nsel) p = 0.f;
      ST[i] = p * (PT[i] - dr);
    }
    const i16x4 da = pack4(ST);
#pragma unroll
    for (int nt = 0; nt < NQ; ++nt)
      dQ[nt] = mfma_16x16x16(da, lds_read_tr16(&Ks[(16 * w + 4 * g + jj) * KST + 16 * nt + 4 * qq]), dQ[nt]);
  }

  // sum the four waves' partial dQ (fixed order) and write bf16
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  if (w > 0) {
#pragma unroll
    for (int nt = 0; nt < NQ; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[((w - 1) * 16 + 4 * g + i) * DQK + 16 * nt + l16] = dQ[nt][i];
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int nt = 0; nt < NQ; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = 4 * g + i;
        const int d = 16 * nt + l16;
        float x = dQ[nt][i];
        x += red[(0 * 16 + hh) * DQK + d];
        x += red[(1 * 16 + hh) * DQK + d];
        x += red[(2 * 16 + hh) * DQK + d];
        if (hh < a.G) a.dq[(t * a.n1 + kvh * a.G + hh) * DQK + d] = f2bf(x * a.scale);
      }
    }
  }
}

QArgs from_dense(const DenseArgs& a) {
  QArgs k{};
  k.q = (const uint16_t*)a.q; k.q_rope = (const uint16_t*)a.q_rope;
  k.k = (const uint16_t*)a.k; k.k_rope = (const uint16_t*)a.k_rope;
  k.v = (const uint16_t*)a.v; k.dy = (const uint16_t*)a.dy;
  k.lse2 = a.lse2; k.drow = a.drow;
  k.dq = (uint16_t*)a.dq; k.dq_rope = (uint16_t*)a.dq_rope;
  k.cu_q = a.cu_q; k.cu_kv = a.cu_kv; k.tiles = a.q_tiles;
  k.batch = a.batch; k.n1 = a.n1; k.n2 = a.n2; k.G = a.G;
  k.d_main = a.d_main; k.d_rope = a.d_rope; k.d_v = a.d_v;
  k.causal = a.causal; k.scale = a.scale; k.scale_log2e = a.scale_log2e;
  return k;
}

}  // namespace

hipError_t launch_dense_bf16(const DenseArgs& a, hipStream_t s) {
  hipError_t e = launch_dense_kv_bf16(a, s);
  if (e != hipSuccess) return e;
  return launch_dense_dq_bf16(a, s);
}

hipError_t launch_dense_dq_bf16(const DenseArgs& a, hipStream_t s) {
  if (a.n_q_tiles == 0) return hipSuccess;
  const QArgs k = from_dense(a);
  const dim3 grid(a.n_q_tiles, a.n1);
  const int dqk = a.d_main + a.d_rope;
  if (dqk == 192 && a.d_v == 128) hipLaunchKernelGGL((dense_dq_kernel<192, 128>), grid, dim3(256), 0, s, k);
  else if (dqk == 128 && a.d_v == 128) hipLaunchKernelGGL((dense_dq_kernel<128, 128>), grid, dim3(256), 0, s, k);
  else if (dqk == 64 && a.d_v == 64) hipLaunchKernelGGL((dense_dq_kernel<64, 64>), grid, dim3(256), 0, s, k);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_selected_dq(const SelArgs& a, int atomic_dkdv, hipStream_t s) {
  if (atomic_dkdv) return hipErrorInvalidValue;
  if (a.T1 == 0) return hipSuccess;
  QArgs k{};
  k.q = (const uint16_t*)a.q; k.k = (const uint16_t*)a.k; k.v = (const uint16_t*)a.v; k.dy = (const uint16_t*)a.dy;
  k.lse2 = a.lse2; k.drow = a.drow; k.dq = (uint16_t*)a.dq;
  k.cu_q = a.cu_q; k.cu_kv = a.cu_kv; k.topk = a.topk;
  k.batch = a.batch; k.n1 = a.n1; k.n2 = a.n2; k.G = a.G;
  k.d_main = a.d_qk; k.d_rope = 0; k.d_v = a.d_v; k.bs = a.bs; k.cnt = a.cnt;
  k.scale = a.scale; k.scale_log2e = a.scale_log2e;
  const dim3 grid((unsigned)(a.T1 * a.n2));
  if (a.d_qk == 192 && a.d_v == 128) hipLaunchKernelGGL((sel_dq_kernel<192, 128>), grid, dim3(256), 0, s, k);
  else if (a.d_qk == 128 && a.d_v == 128) hipLaunchKernelGGL((sel_dq_kernel<128, 128>), grid, dim3(256), 0, s, k);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ab
