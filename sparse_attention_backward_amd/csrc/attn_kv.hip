// KV-major backward: dK and dV, accumulated in registers (bf16 MFMA, fp32 accumulation).
//
// Page "aclnnFlashAttentionUnpaddingScoreGradV3", Formula section (dV = P^T dY,
// dK = dS^T Q / sqrt(d), dkRope = dS^T qRope / sqrt(d)) and page
// "NsaSelectedAttentionGrad", formula section (the same products over the gathered
// selectedKey / selectedValue rows).
//
// One workgroup (4 waves) owns a set of key rows and streams query rows past them in
// tiles of 64 rows:
//   dense:    the key rows are one 64-row tile of a sequence for one KV head; the query
//             rows are the tiles of each of the G query heads of that KV head, from the
//             diagonal tile on when causal.
//   selected: the key rows are one selected block (block_size rows) of one sequence and
//             KV head; the query rows are the G heads of the tokens whose topk rows name
//             the block, read from the inverted index (ascending token order, so the
//             summation order, and hence the result, is fixed).
// Wave w holds key tiles {w, w+4, ...} (16 keys each) of K and V in registers as MFMA B
// operands.  Per 64-row step: S = Q K^T and dP = dY V^T (A operands from LDS),
// P = exp2(S*scale*log2e - lse2), dS = P (dP - drow), then dV += P^T dY and dK += dS^T Q
// with the P / dS C tiles reused directly as A operands and dY / Q read column-wise
// from LDS with ds_read_b64_tr_b16.  No atomics: every key row is owned by one workgroup.
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

constexpr int kRows = 64;  // query rows per step
constexpr int kPad = 8;    // LDS row padding (bf16 elements)

struct KvArgs {
  const uint16_t* q; const uint16_t* q_rope;
  const uint16_t* k; const uint16_t* k_rope;
  const uint16_t* v; const uint16_t* dy;
  const float* lse2; const float* drow;
  uint16_t* dk; uint16_t* dk_rope; uint16_t* dv;
  const int64_t* cu_q; const int64_t* cu_kv;
  const int32_t* tiles;                        // dense: (sequence, key tile)
  const int32_t* blkoff;                       // selected: blocks before each sequence
  const int32_t* offsets; const int32_t* list; // selected: inverted index
  int batch, n1, n2, G, d_main, d_rope, d_v;
  int causal, bs, cnt, nblk_total;
  float scale, scale_log2e;
};

template <int DQK, int DV, int NKT, bool SEL>
__global__ __launch_bounds__(256) void kv_major_kernel(KvArgs a) {
  constexpr int QST = DQK + kPad, YST = DV + kPad;
  constexpr int KS = DQK / 32, VS = DV / 32, NQ = DQK / 16, NV = DV / 16;
  constexpr int QCH = DQK / 8, YCH = DV / 8;  // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint16_t Qs[kRows * QST];
  __shared__ __attribute__((aligned(16))) uint16_t Ys[kRows * YST];
  __shared__ float lse_s[kRows], drow_s[kRows];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4, jj = l16 >> 2, qq = l16 & 3;

  // ---- work unit ------------------------------------------------------------
  int kvh, nk;
  int64_t k0;
  int64_t qs = 0;
  int S1 = 0, kt0 = 0, nqt = 0, qt0 = 0, e_begin = 0, e_end = 0;
  const int TPS = SEL ? (kRows / a.G) : 0;  // selected: tokens per step
  if constexpr (SEL) {
    const int u = blockIdx.x;
    kvh = u / a.nblk_total;
    const int rem = u - kvh * a.nblk_total;
    const int b = seq_of32(a.blkoff, a.batch, rem);
    k0 = a.cu_kv[b] + (int64_t)(rem - a.blkoff[b]) * a.bs;
    nk = a.bs;
    e_begin = a.offsets[u];
    e_end = a.offsets[u + 1];
  } else {
    const int b = a.tiles[2 * blockIdx.x];
    kt0 = a.tiles[2 * blockIdx.x + 1];
    kvh = blockIdx.y;
    const int64_t ks = a.cu_kv[b];
    const int S2 = (int)(a.cu_kv[b + 1] - ks);
    k0 = ks + (int64_t)kt0 * kRows;
    nk = min(kRows, S2 - kt0 * kRows);
    qs = a.cu_q[b];
    S1 = (int)(a.cu_q[b + 1] - qs);
    nqt = (S1 + kRows - 1) / kRows;
    qt0 = a.causal ? kt0 : 0;
    if (qt0 > nqt) qt0 = nqt;
  }

  // ---- resident keys: B operands of S = Q K^T and dP = dY V^T ---------------------
  bf16x8 Kf[NKT][KS], Vf[NKT][VS];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    const int key = 16 * (kt * 4 + w) + l16;
    const bool valid = key < nk;
    const int64_t kr = (k0 + key) * a.n2 + kvh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int d = 32 * s + 8 * g;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (valid) x = ldg16(d < a.d_main ? a.k + kr * a.d_main + d : a.k_rope + kr * a.d_rope + (d - a.d_main));
      Kf[kt][s] = __builtin_bit_cast(bf16x8, x);
    }
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      const int d = 32 * s + 8 * g;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (valid) x = ldg16(a.v + kr * a.d_v + d);
      Vf[kt][s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x4 dK[NKT][NQ], dV[NKT][NV];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) dK[kt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NV; ++n) dV[kt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int nsteps = SEL ? (e_end - e_begin + TPS - 1) / TPS : a.G * (nqt - qt0);
  for (int st = 0; st < nsteps; ++st) {
    int hg = 0, qt = 0, ebase = 0;
    if constexpr (SEL) {
      ebase = e_begin + st * TPS;
    } else {
      hg = st / (nqt - qt0);
      qt = qt0 + (st - hg * (nqt - qt0));
    }
    // query row r of this step -> (token, head) or invalid
    auto row_of = [&](int r, int64_t& t, int& h) -> bool {
      if constexpr (SEL) {
        const int slot = r / a.G;
        const int e = ebase + slot;
        h = kvh * a.G + (r - slot * a.G);
        if (slot >= TPS || e >= e_end) { t = 0; return false; }
        t = a.list[e] / a.cnt;
        return true;
      } else {
        h = kvh * a.G + hg;
        t = qs + qt * kRows + r;
        return qt * kRows + r < S1;
      }
    };

    __syncthreads();  // previous step finished reading Qs / Ys
    for (int idx = tid; idx < kRows * QCH; idx += 256) {
      const int r = idx / QCH, d = 8 * (idx - r * QCH);
      int64_t t; int h;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row_of(r, t, h)) {
        const int64_t qr = t * a.n1 + h;
        x = ldg16(d < a.d_main ? a.q + qr * a.d_main + d : a.q_rope + qr * a.d_rope + (d - a.d_main));
      }
      sts16(&Qs[r * QST + d], x);
    }
    for (int idx = tid; idx < kRows * YCH; idx += 256) {
      const int r = idx / YCH, d = 8 * (idx - r * YCH);
      int64_t t; int h;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row_of(r, t, h)) x = ldg16(a.dy + (t * a.n1 + h) * a.d_v + d);
      sts16(&Ys[r * YST + d], x);
    }
    if (tid < kRows) {
      int64_t t; int h;
      const bool ok = row_of(tid, t, h);
      lse_s[tid] = ok ? a.lse2[t * a.n1 + h] : INFINITY;
      drow_s[tid] = ok ? a.drow[t * a.n1 + h] : 0.f;
    }
    __syncthreads();

    // S = Q K^T, dP = dY V^T for the wave's key tiles (C: lane = key, 4 rows)
    f32x4 S[4][NKT], D[4][NKT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) { S[rt][kt] = f32x4{0.f, 0.f, 0.f, 0.f}; D[rt][kt] = S[rt][kt]; }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 x = lds_read_b128(&Qs[(16 * rt + l16) * QST + 32 * s + 8 * g]);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) S[rt][kt] = mfma_16x16x32(x, Kf[kt][s], S[rt][kt]);
      }
#pragma unroll
      for (int s = 0; s < VS; ++s) {
        const bf16x8 x = lds_read_b128(&Ys[(16 * rt + l16) * YST + 32 * s + 8 * g]);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) D[rt][kt] = mfma_16x16x32(x, Vf[kt][s], D[rt][kt]);
      }
    }
    // P and dS in place
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        const float lse = lse_s[r], dr = drow_s[r];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          float p = __builtin_amdgcn_exp2f(S[rt][kt][i] * a.scale_log2e - lse);
          if constexpr (!SEL) {
            if (a.causal && kt0 * kRows + 16 * (kt * 4 + w) + l16 > qt * kRows + r) p = 0.f;
          }
          D[rt][kt][i] = p * (D[rt][kt][i] - dr);
          S[rt][kt][i] = p;
        }
      }
    }
    // dV += P^T dY, dK += dS^T Q over the two 32-row halves of the step
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 pa[NKT], da[NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        pa[kt] = pack8(S[2 * ks][kt], S[2 * ks + 1][kt]);
        da[kt] = pack8(D[2 * ks][kt], D[2 * ks + 1][kt]);
      }
#pragma unroll
      for (int nt = 0; nt < NV; ++nt) {
        const uint16_t* p = &Ys[(32 * ks + 4 * g + jj) * YST + 16 * nt + 4 * qq];
        const bf16x8 bv = join8(lds_read_tr16(p), lds_read_tr16(p + 16 * YST));
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) dV[kt][nt] = mfma_16x16x32(pa[kt], bv, dV[kt][nt]);
      }
#pragma unroll
      for (int nt = 0; nt < NQ; ++nt) {
        const uint16_t* p = &Qs[(32 * ks + 4 * g + jj) * QST + 16 * nt + 4 * qq];
        const bf16x8 bq = join8(lds_read_tr16(p), lds_read_tr16(p + 16 * QST));
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) dK[kt][nt] = mfma_16x16x32(da[kt], bq, dK[kt][nt]);
      }
    }
  }

  // ---- epilogue: bf16 through LDS, 16-byte stores -----------------------------------
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NQ; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Qs[(16 * w + 4 * g + i) * QST + 16 * nt + l16] = f2bf(dK[kt][nt][i] * a.scale);
#pragma unroll
    for (int nt = 0; nt < NV; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Ys[(16 * w + 4 * g + i) * YST + 16 * nt + l16] = f2bf(dV[kt][nt][i]);
    __syncthreads();
    for (int idx = tid; idx < kRows * QCH; idx += 256) {
      const int r = idx / QCH, d = 8 * (idx - r * QCH);
      const int key = kt * kRows + r;
      if (key < nk) {
        const int64_t kr = (k0 + key) * a.n2 + kvh;
        uint16_t* dst = d < a.d_main ? a.dk + kr * a.d_main + d : a.dk_rope + kr * a.d_rope + (d - a.d_main);
        sts16(dst, *reinterpret_cast<const uint4*>(&Qs[r * QST + d]));
      }
    }
    for (int idx = tid; idx < kRows * YCH; idx += 256) {
      const int r = idx / YCH, d = 8 * (idx - r * YCH);
      const int key = kt * kRows + r;
      if (key < nk) sts16(a.dv + ((k0 + key) * a.n2 + kvh) * a.d_v + d, *reinterpret_cast<const uint4*>(&Ys[r * YST + d]));
    }
  }
}

template <int DQK, int DV, int NKT, bool SEL>
hipError_t launch_kv(const KvArgs& k, dim3 grid, hipStream_t s) {
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((kv_major_kernel<DQK, DV, NKT, SEL>), grid, dim3(256), 0, s, k);
  return hipGetLastError();
}

}  // namespace

bool dense_bf16_supported(int d_qk_total, int d_v) {
  return (d_qk_total == 192 && d_v == 128) || (d_qk_total == 128 && d_v == 128) || (d_qk_total == 64 && d_v == 64);
}

hipError_t launch_dense_kv_bf16(const DenseArgs& a, hipStream_t s) {
  KvArgs k{};
  k.q = (const uint16_t*)a.q; k.q_rope = (const uint16_t*)a.q_rope;
  k.k = (const uint16_t*)a.k; k.k_rope = (const uint16_t*)a.k_rope;
  k.v = (const uint16_t*)a.v; k.dy = (const uint16_t*)a.dy;
  k.lse2 = a.lse2; k.drow = a.drow;
  k.dk = (uint16_t*)a.dk; k.dk_rope = (uint16_t*)a.dk_rope; k.dv = (uint16_t*)a.dv;
  k.cu_q = a.cu_q; k.cu_kv = a.cu_kv; k.tiles = a.kv_tiles;
  k.batch = a.batch; k.n1 = a.n1; k.n2 = a.n2; k.G = a.G;
  k.d_main = a.d_main; k.d_rope = a.d_rope; k.d_v = a.d_v;
  k.causal = a.causal; k.scale = a.scale; k.scale_log2e = a.scale_log2e;
  const dim3 grid(a.n_kv_tiles, a.n2);
  const int dqk = a.d_main + a.d_rope;
  if (dqk == 192 && a.d_v == 128) return launch_kv<192, 128, 1, false>(k, grid, s);
  if (dqk == 128 && a.d_v == 128) return launch_kv<128, 128, 1, false>(k, grid, s);
  if (dqk == 64 && a.d_v == 64) return launch_kv<64, 64, 1, false>(k, grid, s);
  return hipErrorInvalidValue;
}

bool selected_supported(int d_qk, int d_v, int G, int bs) {
  return ((d_qk == 192 && d_v == 128) || (d_qk == 128 && d_v == 128)) && G >= 1 && G <= 16 && bs % 16 == 0 &&
         bs >= 16 && bs <= 128;
}

hipError_t launch_selected_dkdv(const SelArgs& a, hipStream_t s) {
  KvArgs k{};
  k.q = (const uint16_t*)a.q; k.k = (const uint16_t*)a.k; k.v = (const uint16_t*)a.v;
  k.dy = (const uint16_t*)a.dy; k.lse2 = a.lse2; k.drow = a.drow;
  k.dk = (uint16_t*)a.dk; k.dv = (uint16_t*)a.dv;
  k.cu_q = a.cu_q; k.cu_kv = a.cu_kv; k.blkoff = a.blkoff; k.offsets = a.offsets; k.list = a.list;
  k.batch = a.batch; k.n1 = a.n1; k.n2 = a.n2; k.G = a.G;
  k.d_main = a.d_qk; k.d_rope = 0; k.d_v = a.d_v;
  k.bs = a.bs; k.cnt = a.cnt; k.nblk_total = a.nblk_total;
  k.scale = a.scale; k.scale_log2e = a.scale_log2e;
  const dim3 grid((unsigned)(a.n2 * a.nblk_total), 1);
  const bool two = a.bs > 64;
  if (a.d_qk == 192 && a.d_v == 128)
    return two ? launch_kv<192, 128, 2, true>(k, grid, s) : launch_kv<192, 128, 1, true>(k, grid, s);
  if (a.d_qk == 128 && a.d_v == 128)
    return two ? launch_kv<128, 128, 2, true>(k, grid, s) : launch_kv<128, 128, 1, true>(k, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace ab
