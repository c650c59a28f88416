// Kernel argument blocks and launchers (host-callable), shared by the C-ABI layer
// and the kernel translation units.  All pointers are device pointers unless noted.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ab {

// ---- row statistics: lse2 = (m + ln l) * log2(e), ndrow = -rowsum(dY * O) ------
struct PreArgs {
  const void* out;        // [rows, dv] bf16, fp16 or fp32; null: ndrow is not written
  const void* dy;         // [rows, dv]
  const float* smax;      // [rows, 8]
  const float* ssum;      // [rows, 8]
  float* lse2;            // [rows]
  float* ndrow;           // [rows]
  int64_t rows;           // T1 * N1
  int dv;
  int elem;               // element type of out / dy: 0 bf16, 1 fp16, 2 fp32
  const uint4* tab_src;   // the call's tables in pinned host memory (read by the kernel) ...
  uint4* tab_dst;         // ... copied to the start of the workspace: tab_n16 16-byte words
  int64_t tab_n16;
};
hipError_t launch_preprocess(const PreArgs& a, hipStream_t s);

// ---- dense varlen ------------------------------------------------------------
// Masks on the relative position d = j - i of key j and query i (positions in their
// sequence): key j is visible to query i iff lo <= d <= hi.  No mask: lo = -kBandInf,
// hi = kBandInf; causal: hi = off; window of preTokens / nextTokens: lo = off - pre,
// hi = off + next; off = 0 aligns the first query with the first key, off = S2 - S1 the
// last query with the last key.  The schedule (host) and the kernels use these helpers.
constexpr int kBandInf = 1 << 30;
__host__ __device__ inline void dense_band(int lo_rel, int hi_rel, int align, int64_t S1, int64_t S2, int& lo,
                                           int& hi) {
  const int off = align ? (int)(S2 - S1) : 0;
  lo = lo_rel <= -kBandInf ? -kBandInf : lo_rel + off;
  hi = hi_rel >= kBandInf ? kBandInf : hi_rel + off;
}
// Tiles [tlo, thi) of `tile` keys holding a key visible to some query row in [i0, i1) (an empty
// range gives tlo = thi = 0).
__host__ __device__ inline void dense_key_tiles(int lo, int hi, int64_t i0, int64_t i1, int64_t S2, int tile,
                                                int& tlo, int& thi) {
  const int64_t a = i0 + lo > 0 ? i0 + lo : 0, b = (i1 - 1) + hi < S2 - 1 ? (i1 - 1) + hi : S2 - 1;
  if (i1 <= i0 || S2 <= 0 || a > b) { tlo = thi = 0; return; }
  tlo = (int)(a / tile);
  thi = (int)(b / tile) + 1;
}
// Tiles [tlo, thi) of `tile` query rows holding a row that sees some key in [j0, j1).
__host__ __device__ inline void dense_row_tiles(int lo, int hi, int64_t j0, int64_t j1, int64_t S1, int tile,
                                                int& tlo, int& thi) {
  const int64_t a = j0 - hi > 0 ? j0 - hi : 0, b = (j1 - 1) - lo < S1 - 1 ? (j1 - 1) - lo : S1 - 1;
  if (j1 <= j0 || S1 <= 0 || a > b) { tlo = thi = 0; return; }
  tlo = (int)(a / tile);
  thi = (int)(b / tile) + 1;
}

struct DenseArgs {
  const void* q;  const void* q_rope;
  const void* k;  const void* k_rope;
  const void* v;  const void* dy;
  const float* lse2; const float* ndrow;
  void* dq; void* dq_rope; void* dk; void* dk_rope; void* dv;
  void* ds;                 // bf16 dS^T blocks [block][N1][64][64] (stored-dS mode), else null
  const int64_t* cu_q;      // [B+1]
  const int64_t* cu_kv;     // [B+1]
  // stored dS blocks: query tile q (global index qt_base[b] + local tile) has 64-key tiles
  // [qt_kr[2q], qt_kr[2q + 1]), whose blocks start at block qt_blk[q]
  const int32_t* qt_base;   // [B+1] query tiles before each sequence
  const int64_t* qt_blk;    // [query tiles]
  const int32_t* qt_kr;     // [query tiles][2]
  const int32_t* kv_tiles;  // [n_kv_tiles, 6] = (sequence, 128-key tile, KV head, first query tile,
                            //  end query tile, partial slot or -1); sequence -1 = idle slot
  const int32_t* kv_split;  // [n_kv_split, 5] = (sequence, 128-key tile, KV head, first slot, parts)
  void* kv_part;            // fp32 partial dK / dV of split key tiles, 160 KiB per slot
  const int32_t* q_tiles;   // [n_q_tiles, 2]  = (sequence, query tile), heaviest first
  int n_kv_tiles, n_kv_split, n_q_tiles;
  int batch, n1, n2, G;
  int64_t T1, T2;
  int d_main, d_rope, d_v;  // head dims: query/key main part, rope part, value
  float scale, scale_log2e;
  int mask_on;              // a mask applies (causal or window); lo_rel / hi_rel / align as in dense_band
  int lo_rel, hi_rel, align;
};
constexpr int kDenseTile = 64;      // query tile and dS block length of the bf16 dense kernels
constexpr int kDenseKeyTile = 128;  // keys per workgroup of the bf16 dense KV-major kernel
constexpr int kDenseKvPartBytes = 256 * 40 * 16;  // one fp32 partial: 4 waves x 64 lanes x 40 f32x4
bool dense_bf16_supported(int d_main, int d_rope, int d_v);
hipError_t launch_dense_kv_bf16(const DenseArgs& a, hipStream_t s);     // KV-major dK, dV (+ dS when a.ds)
hipError_t launch_dense_kv_combine(const DenseArgs& a, hipStream_t s);  // dK, dV of split key tiles alone
hipError_t launch_dense_dq_from_ds(const DenseArgs& a, hipStream_t s);  // split key tiles + dQ = scale dS K
hipError_t launch_dense_dq_bf16(const DenseArgs& a, hipStream_t s);     // query-major dQ, recomputing S, dP
constexpr int kDenseTileF32 = 64;
hipError_t launch_dense_fp32(const DenseArgs& a, hipStream_t s);

// ---- selected (NSA) ----------------------------------------------------------
struct SelArgs {
  const void* q; const void* k; const void* v; const void* dy;
  const float* lse2; const float* ndrow;
  const int32_t* topk;      // [T1, N2, cnt]
  void* dq; void* dk; void* dv;
  const int64_t* cu_q;      // [B+1]
  const int64_t* cu_kv;     // [B+1]
  const int32_t* blkoff;    // [B+1] running sum of blocks per sequence (S2_b / bs)
  int batch, n1, n2, G, d_qk, d_v, bs, cnt;
  int nblk_total;           // blkoff[B]
  int64_t T1;
  float scale, scale_log2e;
  // inverted index (workspace)
  int32_t* counts;          // [nkeys]      nkeys = n2 * nblk_total
  int32_t* offsets;         // [nkeys + 1]
  int32_t* cursor;          // [nkeys] fill cursors, then the work order of the KV-major kernel
  int32_t* list;            // [T1 * n2 * cnt]  entries t * cnt + slot, sorted per key
  int32_t* sort_scratch;    // [2 * T1 * n2 * cnt]
  int32_t* flag;            // [1] raised on an out-of-range topk id
  void* dq_part;            // [W, cnt, n2] shares of G x d_qk in the element type (chunks ordered as
                            // share_layout.hpp says): each block's share of dQ, for the W query
                            // tokens of the current window, then one share of trash rows
  int64_t T2;
  // query-token windows: the KV-major pass and the dQ reduction run once per window of
  // win_tokens consecutive query tokens, so the share buffer holds one window
  int nwin;                 // number of windows (1: the whole problem at once)
  int64_t win_tokens;       // tokens per window (the last may be shorter)
  int32_t* wofs;            // [n2 * nblk_total, nwin + 1] first list position of each window (nwin > 1)
  float* kvacc;             // fp32 dK / dV accumulators of every (KV head, block) between windows (nwin > 1):
                            // sel_kv_keys(bs) * (d_qk + d_v) floats per (KV head, block), in register order
  int win;                  // current window
  int64_t t0, t1;           // its query tokens [t0, t1)
  int is_f16;               // element type of the tensors and shares: 0 bf16, 1 fp16
};
bool selected_supported(int d_qk, int d_v, int G, int bs);
inline int sel_kv_keys(int bs) { return bs > 64 ? 128 : 64; }  // keys per KV-major workgroup
hipError_t launch_selected_index(const SelArgs& a, hipStream_t s);
hipError_t launch_selected_window_offsets(const SelArgs& a, hipStream_t s);  // wofs from the lists (nwin > 1)
hipError_t launch_selected_kv(const SelArgs& a, hipStream_t s);         // dK, dV and the dQ partials
hipError_t launch_selected_dq_reduce(const SelArgs& a, hipStream_t s);  // dQ = scale * sum of partials

// ---- selected (NSA) forward (KV-major + combine), and the row statistic without attentionOut ----
struct SelFwdArgs {
  const void* q; const void* k; const void* v; const void* dy;  // dy: row-statistic pass only
  const int32_t* topk;      // [T1, N2, cnt]
  const int64_t* cu_q;      // [B+1] (device)
  const int64_t* cu_kv;     // [B+1] (device)
  void* o;                  // forward: O [T1, N1, d_v]
  float* smax; float* ssum; // forward: [T1, N1, 8] softmaxMax, softmaxSum
  const float* lse2;        // row-statistic pass: [T1 * N1] (m + ln l) log2 e
  float* ndrow;             // row-statistic pass: [T1 * N1] -sum_j P_j dP_j
  int32_t* flag;            // raised on an out-of-range topk id (may be null)
  int batch, n1, n2, G, d_qk, d_v, bs, cnt;
  int64_t T1;
  float scale_log2e;
  int is_f16;               // element type: 0 bf16, 1 fp16
  // KV-major forward: the inverted index of the selected backward, and per-entry partials
  const int32_t* blkoff;    // [B+1] blocks before each sequence
  const int32_t* offsets;   // [n2 * nblk_total + 1]
  const int32_t* list;      // entries t * cnt + slot, ascending per key
  const int32_t* sched;     // work order of the keys
  const int32_t* wofs;      // [n2 * nblk_total, nwin + 1] (nwin > 1)
  int nblk_total, nwin, win;
  int64_t t0, t1;           // query tokens of the current window
  void* part_o;             // [W * cnt * n2][d_v / 16][G][16] O_b / l_b of each entry of the window (element type)
  float2* part_ml;          // [W * cnt * n2, G] (m_b, l_b), log2 domain
  float* part_d;            // row statistic: [W * cnt, N1] each entry's sum of P dP per head
};
hipError_t launch_selected_forward_kv(const SelFwdArgs& a, hipStream_t s);       // per-entry partials
hipError_t launch_selected_forward_combine(const SelFwdArgs& a, hipStream_t s);  // O, softmaxMax, softmaxSum
hipError_t launch_selected_drow_kv(const SelFwdArgs& a, hipStream_t s);          // per-entry sums of P dP
hipError_t launch_selected_drow_combine(const SelFwdArgs& a, hipStream_t s);     // ndrow without O

// ---- lightning-indexer backward ------------------------------------------------
struct IdxArgs {
  const void* q;            // [T1, N1, D] bf16
  const void* k;            // [T2, N2, D] bf16
  const void* weights;      // [T1, N1] bf16
  const void* dy;           // [T1, N2, topk] bf16
  const int32_t* indices;   // [T1, N2, topk] key positions in the token's sequence
  void* dq; void* dk; void* dweights;
  float* dk_acc;            // [T2, N2, D] fp32 accumulator of dK
  uint16_t* contrib;        // ordered mode: [units of the window, topk, D] bf16 shares of dK
  const int64_t* cu_q; const int64_t* cu_kv;
  int32_t* flag;            // raised on an out-of-range index
  int batch, n1, n2, G, d, topk;
  int64_t T1, T2;
  int64_t unit0, unit1;     // (token, key head) units t N2 + n2 of this launch
  int atomic;               // 1: dK by fp32 atomics; 0: contributions + ordered reduction
  // inverted index (deterministic mode): keys kvh T2 + j, lists of entries t topk + slot
  const int32_t* offsets; const int32_t* list; const int32_t* wofs;
  int64_t nkeys;
  int nwin, win;
};
bool indexer_supported(int d, int G);
hipError_t launch_indexer_zero(const IdxArgs& a, hipStream_t s);       // dk_acc = 0
hipError_t launch_indexer_qm(const IdxArgs& a, hipStream_t s);         // dQ, dW and the dK shares
hipError_t launch_indexer_dk_reduce(const IdxArgs& a, hipStream_t s);  // deterministic: shares -> dk_acc
hipError_t launch_indexer_dk_cast(const IdxArgs& a, hipStream_t s);    // dk_acc -> dK (bf16)

// ---- misc --------------------------------------------------------------------
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);  // kernel, not a memset node

}  // namespace ab
