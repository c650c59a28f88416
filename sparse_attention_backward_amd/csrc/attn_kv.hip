// KV-major backward on bf16 MFMA with fp32 accumulation.
//
// Page "aclnnFlashAttentionUnpaddingScoreGradV3", Formula section (dV = P^T dY,
// dK = dS^T Q / sqrt(d), dkRope = dS^T qRope / sqrt(d)) and page
// "NsaSelectedAttentionGrad", formula section (the same products over the gathered
// selectedKey / selectedValue rows, plus dQ = dS K / sqrt(d)).
//
// One workgroup (4 waves) owns a set of key rows and streams query rows past them in
// steps of 64 rows:
//   dense:    the key rows are one 64-row tile of a sequence for one KV head; the query
//             rows are the tiles of each of the G query heads of that KV head, from the
//             diagonal tile on when causal.  dK and dV only (dQ has its own kernel).
//   selected: the key rows are one selected block (block_size rows) of one sequence and
//             KV head; the query rows are the G heads of the tokens whose topk rows name
//             the block, read from the inverted index in ascending token order.  Besides
//             dK and dV the workgroup writes, for every (token, slot) it serves, the
//             block's share of dQ -- dS_block K_block, rounded to bf16 -- into a partial
//             buffer that dq_reduce_kernel sums over the slots in a fixed order.
// Wave w holds key tiles {w, w+4} (16 keys each) of K and V as MFMA B operands (dense:
// in registers; selected: in LDS, where the K block also feeds the dQ product).  Per step: S = Q K^T and dP = dY V^T (A operands from LDS),
// P = exp2(S*scale*log2e - lse2), dS = P (dP - drow); dV += P^T dY and dK += dS^T Q with
// the P / dS C tiles reused directly as A operands and dY / Q read column-wise from LDS
// with ds_read_b64_tr_b16; selected: dS^T goes to LDS and dQ^T = K^T dS^T is formed with
// both operands read column-wise (same key permutation on both sides).  LDS tiles are
// unpadded and XOR-swizzled (Swz) so that row and column reads are bank-conflict free.  The next step's rows are fetched into registers
// while the current step computes.  No atomics: every output row has one owner.
#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

constexpr int kRows = 64;  // query rows per step

struct KvArgs {
  const uint16_t* q; const uint16_t* q_rope;
  const uint16_t* k; const uint16_t* k_rope;
  const uint16_t* v; const uint16_t* dy;
  const float* lse2; const float* drow;
  uint16_t* dk; uint16_t* dk_rope; uint16_t* dv;
  uint16_t* dq_part;                           // selected: [T1, N2, cnt, G, d_qk] bf16
  const int64_t* cu_q; const int64_t* cu_kv;
  const int32_t* tiles;                        // dense: (sequence, key tile)
  const int32_t* blkoff;                       // selected: blocks before each sequence
  const int32_t* offsets; const int32_t* list; // selected: inverted index
  int batch, n1, n2, G, d_main, d_rope, d_v;
  int causal, bs, cnt, nblk_total;
  float scale, scale_log2e;
};

template <int DQK, int DV, int NKT, bool SEL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SEL || DQK > 128 ? 1 : 2, SEL || DQK > 128 ? 1 : 2)))
void kv_major_kernel(KvArgs a) {
  using SQ = Swz<DQK>;   // Qs, and the selected K block
  using SY = Swz<DV>;    // Ys, V block
  using SD = Swz<kRows>; // selected: dS^T [key][row]
  constexpr int KS = DQK / 32, VS = DV / 32, NQ = DQK / 16, NV = DV / 16;
  constexpr int QCH = DQK / 8, YCH = DV / 8;  // 16-byte chunks per row
  constexpr int KEYS = 64 * NKT;
  constexpr int NQW = NQ / 4;                 // selected: dQ dim tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t Qs[kRows * DQK];
  __shared__ __attribute__((aligned(16))) uint16_t Ys[kRows * DV];
  __shared__ __attribute__((aligned(16))) uint16_t Ks[SEL ? KEYS * DQK : 8];
  __shared__ __attribute__((aligned(16))) uint16_t Vsl[KEYS * DV];
  __shared__ __attribute__((aligned(16))) uint16_t dSt[SEL ? KEYS * kRows : 8];
  __shared__ float lse_s[kRows], drow_s[kRows];
  __shared__ int ent_s[kRows];                // selected: list value of each row's token, or -1

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
  // K: dense in registers, selected in LDS (the K block is also the A operand of dQ^T);
  // V: in LDS (keeps the dense kernel within 256 registers: two waves per SIMD).
  constexpr int NKR = SEL ? 1 : NKT;
  constexpr int KSR = SEL ? 1 : KS;
  bf16x8 Kf[NKR][KSR];
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
      if constexpr (SEL) sts16(&Ks[SQ::off(key, d)], x);
      else Kf[kt][s] = __builtin_bit_cast(bf16x8, x);
    }
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      const int d = 32 * s + 8 * g;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (valid) x = ldg16(a.v + kr * a.d_v + d);
      sts16(&Vsl[SY::off(key, d)], x);
    }
  }
  auto kfrag = [&](int kt, int s) -> bf16x8 {
    if constexpr (SEL) return lds_read_b128(&Ks[SQ::off(16 * (kt * 4 + w) + l16, 32 * s + 8 * g)]);
    else return Kf[kt][s];
  };
  auto vfrag = [&](int kt, int s) -> bf16x8 {
    return lds_read_b128(&Vsl[SY::off(16 * (kt * 4 + w) + l16, 32 * s + 8 * g)]);
  };

  f32x4 dK[NKT][NQ], dV[NKT][NV];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) dK[kt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NV; ++n) dV[kt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int nsteps = SEL ? (e_end - e_begin + TPS - 1) / TPS : a.G * (nqt - qt0);

  // Row loads: thread tid serves row r = tid / 4 of a step and its 16-byte chunks
  // c = tid % 4 + 4k, so each row needs one (token, head) lookup per thread.  In the
  // selected form the token comes from the inverted index; that list entry is loaded one
  // step ahead so the Q / dY loads of a step never wait on it.
  constexpr int QPT = QCH / 4, YPT = YCH / 4;
  const int my_r = tid >> 2, my_c = tid & 3;
  auto list_entry = [&](int st) -> int {  // selected: list value of row my_r at step st, or -1
    const int slot = my_r / a.G;
    const int e = e_begin + st * TPS + slot;
    return (slot < TPS && e < e_end) ? a.list[e] : -1;
  };
  uint4 pq[QPT], py[YPT];
  float plse = INFINITY, pdrow = 0.f;
  int pent = -1, ent_ahead = -1;
  auto prefetch = [&](int st, int ent) {
    int64_t t = 0;
    int h = 0;
    bool ok;
    if constexpr (SEL) {
      h = kvh * a.G + (my_r - (my_r / a.G) * a.G);
      ok = ent >= 0;
      if (ok) t = ent / a.cnt;
      pent = ent;
    } else {
      const int hg = st / (nqt - qt0);
      const int qt = qt0 + (st - hg * (nqt - qt0));
      h = kvh * a.G + hg;
      t = qs + qt * kRows + my_r;
      ok = qt * kRows + my_r < S1;
    }
    const int64_t qr = t * a.n1 + h;
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int d = 8 * (my_c + 4 * k);
      pq[k] = make_uint4(0, 0, 0, 0);
      if (ok) pq[k] = ldg16(d < a.d_main ? a.q + qr * a.d_main + d : a.q_rope + qr * a.d_rope + (d - a.d_main));
    }
#pragma unroll
    for (int k = 0; k < YPT; ++k) {
      py[k] = make_uint4(0, 0, 0, 0);
      if (ok) py[k] = ldg16(a.dy + qr * a.d_v + 8 * (my_c + 4 * k));
    }
    if (my_c == 0) {
      plse = ok ? a.lse2[qr] : INFINITY;
      pdrow = ok ? a.drow[qr] : 0.f;
    }
  };

  if (nsteps > 0) {
    if constexpr (SEL) {
      prefetch(0, list_entry(0));
      ent_ahead = nsteps > 1 ? list_entry(1) : -1;
    } else {
      prefetch(0, -1);
    }
  }
  for (int st = 0; st < nsteps; ++st) {
    __syncthreads();  // every wave is done with the previous step's LDS tiles
#pragma unroll
    for (int k = 0; k < QPT; ++k) sts16(&Qs[SQ::off(my_r, 8 * (my_c + 4 * k))], pq[k]);
#pragma unroll
    for (int k = 0; k < YPT; ++k) sts16(&Ys[SY::off(my_r, 8 * (my_c + 4 * k))], py[k]);
    if (my_c == 0) {
      lse_s[my_r] = plse;
      drow_s[my_r] = pdrow;
      if constexpr (SEL) ent_s[my_r] = pent;
    }
    __syncthreads();
    if constexpr (SEL) {
      if (st + 1 < nsteps) {
        const int ent = ent_ahead;
        ent_ahead = st + 2 < nsteps ? list_entry(st + 2) : -1;
        prefetch(st + 1, ent);
      }
    } else {
      if (st + 1 < nsteps) prefetch(st + 1, -1);
    }

    // S = Q K^T, dP = dY V^T for the wave's key tiles (C: lane = key, 4 rows).
    // Items i = (k-step gi, row tile rt) with gi < KS for S and KS <= gi for dP; the A
    // fragment of item i + PD1 is read from LDS while item i's MFMAs issue.
    constexpr int NI1 = 4 * (KS + VS), PD1 = SEL ? 6 : 4;
    f32x4 S[4][NKT], D[4][NKT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) { S[rt][kt] = f32x4{0.f, 0.f, 0.f, 0.f}; D[rt][kt] = S[rt][kt]; }
    auto a1 = [&](int i) -> bf16x8 {
      const int gi = i >> 2, rt = i & 3;
      return gi < KS ? lds_read_b128(&Qs[SQ::off(16 * rt + l16, 32 * gi + 8 * g)])
                     : lds_read_b128(&Ys[SY::off(16 * rt + l16, 32 * (gi - KS) + 8 * g)]);
    };
    auto b1 = [&](int gi, int kt) -> bf16x8 { return gi < KS ? kfrag(kt, gi) : vfrag(kt, gi - KS); };
    bf16x8 ring1[PD1], bcur[NKT], bnext[NKT];
#pragma unroll
    for (int i = 0; i < PD1; ++i) ring1[i] = a1(i);
    // B fragments from LDS (selected K, and V) are read one k-step ahead; the dense K
    // fragments are used straight from registers.
    constexpr int G0 = SEL ? 0 : KS;  // first k-step whose B fragment comes from LDS
    if (G0 < KS + VS) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) bcur[kt] = b1(G0, kt);
    }
#pragma unroll
    for (int i = 0; i < NI1; ++i) {
      const int gi = i >> 2, rt = i & 3;
      if (rt == 0 && gi >= G0 && gi + 1 < KS + VS) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) bnext[kt] = b1(gi + 1, kt);
      }
      const bf16x8 x = ring1[i % PD1];
      if (i + PD1 < NI1) ring1[i % PD1] = a1(i + PD1);
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const bf16x8 bk = gi < G0 ? kfrag(kt, gi < KS ? gi : 0) : bcur[kt];
        if (gi < KS) S[rt][kt] = mfma_16x16x32(x, bk, S[rt][kt]);
        else D[rt][kt] = mfma_16x16x32(x, bk, D[rt][kt]);
      }
      if (rt == 3 && gi >= G0) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) bcur[kt] = bnext[kt];
      }
    }
    // P and dS in place
    int qt = 0;
    if constexpr (!SEL) { const int hg = st / (nqt - qt0); qt = qt0 + (st - hg * (nqt - qt0)); }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        const float lse = lse_s[r], dr = drow_s[r];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          const int key = 16 * (kt * 4 + w) + l16;
          float p = __builtin_amdgcn_exp2f(S[rt][kt][i] * a.scale_log2e - lse);
          if constexpr (SEL) {
            if (key >= nk) p = 0.f;
          } else {
            if (a.causal && kt0 * kRows + key > qt * kRows + r) p = 0.f;
          }
          D[rt][kt][i] = p * (D[rt][kt][i] - dr);
          S[rt][kt][i] = p;
        }
      }
    }
    if constexpr (SEL) {
      // dS^T [key][row] for the dQ product (4 consecutive rows per lane: one 8-byte store)
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          *reinterpret_cast<i16x4*>(&dSt[SD::off(16 * (kt * 4 + w) + l16, 16 * rt + 4 * g)]) = pack4(D[rt][kt]);
    }
    // dV += P^T dY, dK += dS^T Q over the two 32-row halves of the step.  Items
    // i = (half ks, output tile j): j < NV feeds dV from dY, else dK from Q; the column
    // fragments (two transposed reads each) run PD2 items ahead of the MFMAs.
    bf16x8 pa[2][NKT], da[2][NKT];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        pa[ks][kt] = pack8(S[2 * ks][kt], S[2 * ks + 1][kt]);
        da[ks][kt] = pack8(D[2 * ks][kt], D[2 * ks + 1][kt]);
      }
    constexpr int NJ = NV + NQ, NI2 = 2 * NJ, PD2 = SEL ? 6 : 4;
    auto b2 = [&](int i) -> bf16x8 {
      const int ks = i / NJ, j = i - (i / NJ) * NJ;
      const int r = 32 * ks + 4 * g + jj;
      if (j < NV) {
        const int col = 16 * j + 4 * qq;
        return join8(lds_read_tr16(&Ys[SY::off(r, col)]), lds_read_tr16(&Ys[SY::off(r + 16, col)]));
      }
      const int col = 16 * (j - NV) + 4 * qq;
      return join8(lds_read_tr16(&Qs[SQ::off(r, col)]), lds_read_tr16(&Qs[SQ::off(r + 16, col)]));
    };
    bf16x8 ring2[PD2];
#pragma unroll
    for (int i = 0; i < PD2; ++i) ring2[i] = b2(i);
#pragma unroll
    for (int i = 0; i < NI2; ++i) {
      const int ks = i / NJ, j = i - (i / NJ) * NJ;
      const bf16x8 bv = ring2[i % PD2];
      if (i + PD2 < NI2) ring2[i % PD2] = b2(i + PD2);
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        if (j < NV) dV[kt][j] = mfma_16x16x32(pa[ks][kt], bv, dV[kt][j]);
        else dK[kt][j - NV] = mfma_16x16x32(da[ks][kt], bv, dK[kt][j - NV]);
      }
    }
    if constexpr (SEL) {
      __syncthreads();  // dS^T complete
      // dQ^T (dims x rows) = K^T dS^T over the block's keys; wave w takes NQW dim tiles
      f32x4 acc[NQW][4];
#pragma unroll
      for (int dt = 0; dt < NQW; ++dt)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      auto ld3 = [&](int ks, bf16x8* bs_, bf16x8* ak) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const int r = 32 * ks + 4 * g + jj, col = 16 * rt + 4 * qq;
          bs_[rt] = join8(lds_read_tr16(&dSt[SD::off(r, col)]), lds_read_tr16(&dSt[SD::off(r + 16, col)]));
        }
#pragma unroll
        for (int dt = 0; dt < NQW; ++dt) {
          const int r = 32 * ks + 4 * g + jj, col = 16 * (w * NQW + dt) + 4 * qq;
          ak[dt] = join8(lds_read_tr16(&Ks[SQ::off(r, col)]), lds_read_tr16(&Ks[SQ::off(r + 16, col)]));
        }
      };
      bf16x8 bs3[2][4], ak3[2][NQW];
      ld3(0, bs3[0], ak3[0]);
#pragma unroll
      for (int ks = 0; ks < KEYS / 32; ++ks) {
        if (ks + 1 < KEYS / 32) ld3(ks + 1, bs3[(ks + 1) & 1], ak3[(ks + 1) & 1]);
#pragma unroll
        for (int dt = 0; dt < NQW; ++dt)
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) acc[dt][rt] = mfma_16x16x32(ak3[ks & 1][dt], bs3[ks & 1][rt], acc[dt][rt]);
      }
      // C tile: lane holds row 16rt + l16, dims 16(w*NQW+dt) + 4g .. +3 -> one 8-byte store
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int r = 16 * rt + l16;
        const int ent = ent_s[r];
        if (ent >= 0) {
          const int64_t t = ent / a.cnt, sl = ent - t * a.cnt;
          uint16_t* dst = a.dq_part + (((t * a.n2 + kvh) * a.cnt + sl) * a.G + (r - (r / a.G) * a.G)) * DQK;
#pragma unroll
          for (int dt = 0; dt < NQW; ++dt)
            *reinterpret_cast<i16x4*>(dst + 16 * (w * NQW + dt) + 4 * g) = pack4(acc[dt][rt]);
        }
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
      for (int i = 0; i < 4; ++i) Qs[SQ::off(16 * w + 4 * g + i, 16 * nt + l16)] = f2bf(dK[kt][nt][i] * a.scale);
#pragma unroll
    for (int nt = 0; nt < NV; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Ys[SY::off(16 * w + 4 * g + i, 16 * nt + l16)] = f2bf(dV[kt][nt][i]);
    __syncthreads();
    for (int idx = tid; idx < kRows * QCH; idx += 256) {
      const int r = idx / QCH, d = 8 * (idx - r * QCH);
      const int key = kt * kRows + r;
      if (key < nk) {
        const int64_t kr = (k0 + key) * a.n2 + kvh;
        uint16_t* dst = d < a.d_main ? a.dk + kr * a.d_main + d : a.dk_rope + kr * a.d_rope + (d - a.d_main);
        sts16(dst, *reinterpret_cast<const uint4*>(&Qs[SQ::off(r, d)]));
      }
    }
    for (int idx = tid; idx < kRows * YCH; idx += 256) {
      const int r = idx / YCH, d = 8 * (idx - r * YCH);
      const int key = kt * kRows + r;
      if (key < nk) sts16(a.dv + ((k0 + key) * a.n2 + kvh) * a.d_v + d, *reinterpret_cast<const uint4*>(&Ys[SY::off(r, d)]));
    }
  }
}

// dQ[t, kvh*G + g, :] = scale * sum over slots of the bf16 partials, slots in order.
// One wave per (token, KV head); each lane owns 8-element chunks of the G x DQK block.
// A slot whose topk id is out of range was never written and is skipped.
template <int DQK>
__global__ __launch_bounds__(256) void dq_reduce_kernel(const uint16_t* part, uint16_t* dq, int64_t pairs, int n2,
                                                        int n1, int G, int cnt, float scale, const int32_t* topk,
                                                        const int64_t* cu_q, const int32_t* blkoff, int batch) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= pairs) return;
  const int64_t t = pair / n2;
  const int kvh = (int)(pair - t * n2);
  const int b = seq_of(cu_q, batch, t);
  const int nblk = blkoff[b + 1] - blkoff[b];
  const int chunks = G * DQK / 8;
  const uint16_t* src = part + pair * (int64_t)cnt * G * DQK;
  uint16_t* out = dq + (t * n1 + (int64_t)kvh * G) * DQK;
  for (int c0 = lane; c0 < chunks; c0 += 64 * 4) {
    float acc[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[u][j] = 0.f;
    for (int sl = 0; sl < cnt; ++sl) {
      const int id = topk[pair * cnt + sl];
      if (id < 0 || id >= nblk) continue;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + 64 * u;
        if (c < chunks) {
          const uint4 x = ldg16(src + (int64_t)sl * G * DQK + 8 * c);
          const uint32_t xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[u][2 * j] += __uint_as_float(xv[j] << 16);
            acc[u][2 * j + 1] += __uint_as_float(xv[j] & 0xffff0000u);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + 64 * u;
      if (c < chunks) {
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = (uint32_t)f2bf(acc[u][2 * j] * scale) | ((uint32_t)f2bf(acc[u][2 * j + 1] * scale) << 16);
        sts16(out + 8 * c, make_uint4(o[0], o[1], o[2], o[3]));
      }
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

bool selected_supported(int d_qk, int d_v, int G, int bs) {
  return ((d_qk == 192 && d_v == 128) || (d_qk == 128 && d_v == 128)) && G >= 1 && G <= 16 && bs % 16 == 0 &&
         bs >= 16 && bs <= 128;
}

hipError_t launch_selected_dkdv(const SelArgs& a, hipStream_t s) {
  KvArgs k{};
  k.q = (const uint16_t*)a.q; k.k = (const uint16_t*)a.k; k.v = (const uint16_t*)a.v;
  k.dy = (const uint16_t*)a.dy; k.lse2 = a.lse2; k.drow = a.drow;
  k.dk = (uint16_t*)a.dk; k.dv = (uint16_t*)a.dv; k.dq_part = (uint16_t*)a.dq_part;
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

hipError_t launch_selected_dq_reduce(const SelArgs& a, hipStream_t s) {
  const int64_t pairs = a.T1 * a.n2;
  if (pairs == 0) return hipSuccess;
  const dim3 grid((unsigned)((pairs + 3) / 4)), block(256);
  if (a.d_qk == 192)
    hipLaunchKernelGGL(dq_reduce_kernel<192>, grid, block, 0, s, (const uint16_t*)a.dq_part, (uint16_t*)a.dq, pairs,
                       a.n2, a.n1, a.G, a.cnt, a.scale, a.topk, a.cu_q, a.blkoff, a.batch);
  else if (a.d_qk == 128)
    hipLaunchKernelGGL(dq_reduce_kernel<128>, grid, block, 0, s, (const uint16_t*)a.dq_part, (uint16_t*)a.dq, pairs,
                       a.n2, a.n1, a.G, a.cnt, a.scale, a.topk, a.cu_q, a.blkoff, a.batch);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ab
