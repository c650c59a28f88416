// C-ABI layer: parameter validation, workspace layout, schedule tables, launches.
//
// The two-phase shape (workspace-size query that validates, then execute with a
// caller-owned workspace on a stream) follows the calling convention that pages
// "aclnnFlashAttentionUnpaddingScoreGradV3", "aclnnMoeTokenPermuteGrad" and the others
// describe for their operators; the constraint checks restate the constraint lists of
// the dense page and of page "NsaSelectedAttentionGrad".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/attn_bwd.h"
#include "kernels.hpp"

namespace {

using namespace ab;

constexpr int64_t kDenseMaxT = 1 << 20;      // dense constraints: T in 1..1M
constexpr int64_t kSelMaxT = 2 << 20;        // selected constraints: T1, T2 in 1..2M
constexpr int64_t kSelMaxS = 128 << 10;      // selected constraints: S in 1..128K
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int B = 0, G = 0;
  int64_t T1 = 0, T2 = 0;
  std::vector<int64_t> cuq, cukv;  // sequence offsets: the caller's (TND) or derived (BSND)
  // dense schedule
  std::vector<int32_t> kv_tiles, kv_split, q_tiles;
  std::vector<int32_t> qt_base, qt_kr;  // query tiles before each sequence; key-tile range of each
  std::vector<int64_t> qt_blk;          // first stored dS block of each query tile
  int64_t ds_blocks = 0;
  int lo_rel = -kBandInf, hi_rel = kBandInf;  // dense mask (dense_band); +-kBandInf: unbounded
  int kv_slots = 0;       // fp32 partial slots of split key tiles
  bool dense_ds = false;  // dQ from stored dS tiles (else recomputed)
  // selected
  std::vector<int32_t> blkoff;
  int nblk_total = 0;
  int64_t entries = 0;
  int nwin = 1;              // windows of query tokens (dQ shares of one window in the workspace)
  int64_t win_tokens = 0;
  bool idx_atomic = false;    // indexer: dK by fp32 atomics (asked for, non-deterministic)
  // workspace layout (byte offsets)
  size_t off_cu_q = 0, off_cu_kv = 0, off_tab1 = 0, off_tab2 = 0, table_bytes = 0;
  size_t off_lse2 = 0, off_ndrow = 0, off_ml = 0;
  size_t off_counts = 0, off_offsets = 0, off_cursor = 0, off_list = 0, off_scratch = 0, off_flag = 0;
  size_t off_dq_part = 0, off_wofs = 0, off_kvacc = 0, off_dkacc = 0, off_contrib = 0;
  size_t off_qt_base = 0, off_qt_blk = 0, off_qt_kr = 0, off_ds = 0, off_kvsplit = 0, off_kvpart = 0;
  size_t total = 0;
};

constexpr int kXcds = 8;                          // workgroups are dealt to the XCDs round-robin
constexpr int kCus = 256;                         // compute units (sets the key-tile split size only)
constexpr uint64_t kDenseDsAutoMax = 8ull << 30;  // stored dS above this size: recompute instead
// Selected: the dQ shares of one window take at most this much workspace.  Windows cost time
// (per window every block's K / V is loaded again and its fp32 dK / dV sums are saved and
// restored; with skewed ids each window's longest list runs alone), so they are made as long
// as the cap allows; the caller can ask for shorter ones (sel_window_tokens).
constexpr uint64_t kSelShareMax = 64ull << 30;
constexpr uint64_t kIdxContribMax = 8ull << 30;  // indexer, ordered dK: bf16 dK shares of one window at most

// Dense schedule tables.
//  * Work items of the KV-major kernel: (sequence, 128-key tile, KV head, query-tile range,
//    partial slot).  A key tile's query tiles (from its diagonal on when causal) form one
//    range, or, when that is more than about 4/5 of a CU's fair share of the whole
//    launch, several ranges whose fp32 partials the dQ launch adds first (in range order).
//    The items of one (sequence, KV head) read the same query rows, so each such group
//    goes to one XCD (groups dealt to the least loaded XCD, largest first) and its items
//    share that XCD's L2.  Within an XCD items run heaviest first.  Slot p of the launch
//    belongs to XCD p % 8; slots an XCD does not need are idle (-1).  The dealing and
//    the split affect speed only, never results.
//  * Split tiles (sequence, 128-key tile, KV head, first slot, ranges) for the combine.
//  * Query tiles (sequence, 64-row query tile), heaviest first.
//  * ds_base: (query tile, 64-key tile) blocks before each sequence (stored-dS layout).
void plan_dense_schedule(const attn_bwd_problem_t* p, Plan& pl) {
  const int B = pl.B;
  const int64_t* cq = pl.cuq.data();
  const int64_t* ck = pl.cukv.data();
  struct W { int64_t work; int32_t b, tile, kvh, qa, qb, slot, part, group; };
  struct T { int32_t b, tile, kvh, qlo, qhi; };
  std::vector<T> tiles;
  std::vector<W> qv;
  int64_t total = 0;
  pl.qt_base.assign(B + 1, 0);
  pl.qt_blk.clear();
  pl.qt_kr.clear();
  pl.ds_blocks = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t S1 = cq[b + 1] - cq[b], S2 = ck[b + 1] - ck[b];
    const int64_t nqt = (S1 + kDenseTile - 1) / kDenseTile;
    const int64_t nkt2 = (S2 + kDenseKeyTile - 1) / kDenseKeyTile;
    int lo, hi;
    dense_band(pl.lo_rel, pl.hi_rel, p->mask_align, S1, S2, lo, hi);
    pl.qt_base[b + 1] = pl.qt_base[b] + (int32_t)nqt;
    // per query tile: the 64-key tiles with a visible key, and their stored dS blocks
    for (int64_t t = 0; t < nqt; ++t) {
      int klo, khi;
      dense_key_tiles(lo, hi, kDenseTile * t, std::min<int64_t>(kDenseTile * (t + 1), S1), S2, kDenseTile, klo, khi);
      pl.qt_blk.push_back(pl.ds_blocks);
      pl.qt_kr.push_back(klo);
      pl.qt_kr.push_back(khi);
      pl.ds_blocks += khi - klo;
      qv.push_back({khi - klo, b, (int32_t)t, 0, 0, 0, 0, 0, 0});
    }
    // per 128-key tile and KV head: the query tiles with a row that sees one of its keys
    for (int h = 0; h < p->n2; ++h)
      for (int64_t t = 0; t < nkt2; ++t) {
        int qlo, qhi;
        dense_row_tiles(lo, hi, kDenseKeyTile * t, std::min<int64_t>(kDenseKeyTile * (t + 1), S2), S1, kDenseTile, qlo,
                        qhi);
        tiles.push_back({b, (int32_t)t, h, (int32_t)qlo, (int32_t)qhi});
        total += (int64_t)(qhi - qlo) * pl.G;
      }
  }
  // Split size in query tiles: about 4/5 of a CU's share of all steps (a steady-state sweep of
  // 1/2 .. 2 shares on the dense workload: longer ranges stretch the KV-major tail, shorter ones
  // add split tiles whose partials the dQ launch must add).  The ranges are cut at
  // the same query tiles for every key tile of a (sequence, KV head) -- counted from the last
  // query tile down -- so that the parts that run together walk the same query rows and share
  // them in the L2.
  const int64_t target = std::max<int64_t>(2 * pl.G, (4 * total + 5 * kCus - 1) / (5 * kCus));
  const int64_t qchunk = std::max<int64_t>(1, target / pl.G);
  std::vector<std::vector<W>> groups;  // per (sequence, KV head)
  std::vector<int64_t> gwork;
  pl.kv_split.clear();
  pl.kv_slots = 0;
  for (size_t i = 0; i < tiles.size(); ++i) {
    const T& t = tiles[i];
    if (i == 0 || t.b != tiles[i - 1].b || t.kvh != tiles[i - 1].kvh) { groups.emplace_back(); gwork.push_back(0); }
    const int64_t nq = t.qhi - t.qlo;
    const int64_t parts = nq > qchunk ? (nq + qchunk - 1) / qchunk : 1;
    const int32_t slot0 = parts > 1 ? pl.kv_slots : -1;
    if (parts > 1) {
      pl.kv_split.insert(pl.kv_split.end(), {t.b, t.tile, t.kvh, slot0, (int32_t)parts});
      pl.kv_slots += (int)parts;
    }
    for (int64_t q = 0; q < parts; ++q) {
      const int32_t qb = (int32_t)(t.qhi - q * qchunk);
      const int32_t qa = parts > 1 ? (int32_t)std::max<int64_t>(t.qlo, qb - qchunk) : (int32_t)t.qlo;
      const int64_t work = std::max<int64_t>((int64_t)(qb - qa) * pl.G, 1);
      groups.back().push_back({work, t.b, t.tile, t.kvh, qa, qb, parts > 1 ? slot0 + (int32_t)q : -1, (int32_t)q,
                               (int32_t)(groups.size() - 1)});
      gwork.back() += work;
    }
  }
  std::vector<size_t> order(groups.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) { return gwork[x] > gwork[y]; });
  std::vector<std::vector<W>> bins(kXcds);
  std::vector<int64_t> load(kXcds, 0);
  for (size_t gi : order) {
    const int x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    load[x] += gwork[gi];
    bins[x].insert(bins[x].end(), groups[gi].begin(), groups[gi].end());
  }
  size_t rounds = 0;
  // longest first; among equal lengths, the parts of one group and one range together
  for (auto& bin : bins) {
    std::stable_sort(bin.begin(), bin.end(), [](const W& x, const W& y) {
      if (x.work != y.work) return x.work > y.work;
      if (x.group != y.group) return x.group < y.group;
      return x.part < y.part;
    });
    rounds = std::max(rounds, bin.size());
  }
  pl.kv_tiles.clear();
  for (size_t r = 0; r < rounds; ++r)
    for (int x = 0; x < kXcds; ++x) {
      if (r < bins[x].size()) {
        const W& t = bins[x][r];
        pl.kv_tiles.insert(pl.kv_tiles.end(), {t.b, t.tile, t.kvh, t.qa, t.qb, t.slot});
      } else {
        pl.kv_tiles.insert(pl.kv_tiles.end(), {-1, 0, 0, 0, 0, -1});
      }
    }
  std::stable_sort(qv.begin(), qv.end(), [](const W& x, const W& y) { return x.work > y.work; });
  for (auto& x : qv) { pl.q_tiles.push_back(x.b); pl.q_tiles.push_back(x.tile); }
  const uint64_t ds_bytes = (uint64_t)pl.ds_blocks * p->n1 * kDenseTile * kDenseTile * 2;
  pl.dense_ds = p->dtype == ATTN_BF16 &&
                (p->dense_dq_mode == 1 || (p->dense_dq_mode == 0 && ds_bytes <= kDenseDsAutoMax));
}

attn_status_t validate_and_plan(const attn_bwd_problem_t* p, Plan& pl) {
  if (!p) return ATTN_ERR_NULLPTR;
  if (p->op != ATTN_OP_DENSE && p->op != ATTN_OP_SELECTED && p->op != ATTN_OP_SELECTED_FWD && p->op != ATTN_OP_INDEXER)
    return ATTN_ERR_INVALID;
  if (p->batch < 1) return ATTN_ERR_INVALID;
  const int B = p->batch;
  if (p->layout == ATTN_LAYOUT_TND) {
    if (!p->cu_seqlens_q || !p->cu_seqlens_kv) return ATTN_ERR_NULLPTR;
    if (p->seq_len_q != 0 || p->seq_len_kv != 0) return ATTN_ERR_INVALID;
    pl.cuq.assign(p->cu_seqlens_q, p->cu_seqlens_q + B + 1);
    pl.cukv.assign(p->cu_seqlens_kv, p->cu_seqlens_kv + B + 1);
  } else if (p->layout == ATTN_LAYOUT_BSND) {
    // [B, S, N, D]: every sequence has seq_len_q queries and seq_len_kv keys, back to back --
    // the TND layout with equal lengths (layouts of the selected and indexer pages)
    if (p->op == ATTN_OP_DENSE) return ATTN_ERR_INVALID;  // the dense page takes TND only
    if (p->cu_seqlens_q || p->cu_seqlens_kv) return ATTN_ERR_INVALID;
    if (p->seq_len_q < 0 || p->seq_len_kv < 0 || p->seq_len_q > (int64_t(1) << 40) / B ||
        p->seq_len_kv > (int64_t(1) << 40) / B)
      return ATTN_ERR_INVALID;
    pl.cuq.resize(B + 1);
    pl.cukv.resize(B + 1);
    for (int b = 0; b <= B; ++b) {
      pl.cuq[b] = (int64_t)b * p->seq_len_q;
      pl.cukv[b] = (int64_t)b * p->seq_len_kv;
    }
  } else {
    return ATTN_ERR_INVALID;
  }
  const int64_t* cq = pl.cuq.data();
  const int64_t* ck = pl.cukv.data();
  if (cq[0] != 0 || ck[0] != 0) return ATTN_ERR_INVALID;
  for (int b = 0; b < B; ++b)
    if (cq[b + 1] < cq[b] || ck[b + 1] < ck[b]) return ATTN_ERR_INVALID;
  if (p->n1 < 1 || p->n2 < 1 || p->n1 % p->n2 != 0) return ATTN_ERR_INVALID;
  if (p->d_qk < 1 || (p->d_v < 1 && p->op != ATTN_OP_INDEXER) || p->d_rope < 0) return ATTN_ERR_INVALID;
  if (!std::isfinite(p->scale)) return ATTN_ERR_INVALID;
  if ((p->causal != 0 && p->causal != 1) || (p->band != 0 && p->band != 1) ||
      (p->mask_align != 0 && p->mask_align != 1) || (p->deterministic != 0 && p->deterministic != 1) ||
      (p->dkdv_atomic != 0 && p->dkdv_atomic != 1))
    return ATTN_ERR_INVALID;
  pl.B = B;
  pl.G = p->n1 / p->n2;
  pl.T1 = cq[B];
  pl.T2 = ck[B];

  if (p->op == ATTN_OP_DENSE) {
    if (p->dtype == ATTN_FP16) return ATTN_ERR_UNSUPPORTED;
    if (p->dtype != ATTN_BF16 && p->dtype != ATTN_FP32) return ATTN_ERR_INVALID;
    // D of query / key and of value / dy: multiples of 8, value D <= query D; D <= 768; N <= 256
    if (p->d_qk % 8 || p->d_v % 8 || p->d_rope % 8) return ATTN_ERR_INVALID;
    if (p->d_v > p->d_qk) return ATTN_ERR_INVALID;
    if (p->d_qk + p->d_rope > 768 || p->n1 > 256) return ATTN_ERR_INVALID;
    if (pl.T1 > kDenseMaxT || pl.T2 > kDenseMaxT) return ATTN_ERR_INVALID;
    // masks on the relative position: causal (aligned top-left or bottom-right when the
    // lengths differ) or a window of pre_tokens / next_tokens around the aligned diagonal
    if (p->causal && p->band) return ATTN_ERR_INVALID;
    if (p->band) {
      if (p->pre_tokens < -kBandInf || p->pre_tokens > kBandInf || p->next_tokens < -kBandInf ||
          p->next_tokens > kBandInf || p->pre_tokens + p->next_tokens < 0)
        return ATTN_ERR_INVALID;
      pl.lo_rel = p->pre_tokens >= kBandInf ? -kBandInf : (int)-p->pre_tokens;
      pl.hi_rel = p->next_tokens >= kBandInf ? kBandInf : (int)p->next_tokens;
    } else if (p->pre_tokens != 0 || p->next_tokens != 0) {
      return ATTN_ERR_INVALID;
    } else if (p->causal) {
      pl.lo_rel = -kBandInf;
      pl.hi_rel = 0;
    }
    const int dqk = p->d_qk + p->d_rope;
    if (p->dtype == ATTN_BF16 && !dense_bf16_supported(p->d_qk, p->d_rope, p->d_v)) return ATTN_ERR_UNSUPPORTED;
    if (p->dtype == ATTN_FP32 && (dqk > 256 || p->d_v > 256)) return ATTN_ERR_UNSUPPORTED;
    if (p->dense_dq_mode < 0 || p->dense_dq_mode > 2 || p->sel_window_tokens != 0 || p->dkdv_atomic != 0)
      return ATTN_ERR_INVALID;
    plan_dense_schedule(p, pl);
  } else if (p->op == ATTN_OP_INDEXER) {
    // lightning-indexer backward (readings of the page's lost shape table: bf16, D = 128,
    // G <= 64, topK key tokens of the token's own sequence, S up to 128K, B up to 1024)
    if (p->dtype != ATTN_BF16) return p->dtype == ATTN_FP16 || p->dtype == ATTN_FP32 ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_INVALID;
    if (p->d_rope != 0 || p->causal != 0 || p->dense_dq_mode != 0 || p->band != 0 || p->mask_align != 0 ||
        p->pre_tokens != 0 || p->next_tokens != 0 || p->d_v != 0 || p->block_size != 1)
      return ATTN_ERR_INVALID;
    pl.idx_atomic = p->dkdv_atomic != 0 && p->deterministic == 0;
    if (B > 1024 || p->n1 > 128 || pl.G > 64) return ATTN_ERR_INVALID;
    const int topk = p->block_count;
    if (topk < 1 || topk > kSelMaxS) return ATTN_ERR_INVALID;
    pl.blkoff.assign(B + 1, 0);
    for (int b = 0; b < B; ++b) {
      const int64_t S1 = cq[b + 1] - cq[b], S2 = ck[b + 1] - ck[b];
      if (S1 > kSelMaxS || S2 > kSelMaxS) return ATTN_ERR_INVALID;
      if (S1 > 0 && S2 < topk) return ATTN_ERR_INVALID;  // S_K from topK up
      pl.blkoff[b + 1] = (int32_t)ck[b + 1];  // one index = one key token
    }
    pl.nblk_total = (int)pl.T2;
    if (!indexer_supported(p->d_qk, pl.G)) return ATTN_ERR_UNSUPPORTED;
    pl.entries = pl.T1 * p->n2 * topk;
    if (pl.entries >= (int64_t(1) << 31) || (int64_t)p->n2 * pl.T2 >= (int64_t(1) << 31)) return ATTN_ERR_UNSUPPORTED;
    // deterministic mode: the fp32 dK shares of one window of query tokens take at most
    // kIdxContribMax; windows of equal length but the last
    if (p->sel_window_tokens < 0) return ATTN_ERR_INVALID;
    const uint64_t per_token = (uint64_t)p->n2 * topk * p->d_qk * 2;
    int64_t w = std::max<int64_t>(1, (int64_t)(kIdxContribMax / per_token));
    if (p->sel_window_tokens > 0) w = std::min<int64_t>(w, p->sel_window_tokens);
    pl.nwin = (int)std::max<int64_t>(1, (pl.T1 + w - 1) / w);
    pl.win_tokens = std::max<int64_t>(1, (pl.T1 + pl.nwin - 1) / pl.nwin);
  } else {
    // selected backward and forward: BFLOAT16 or FLOAT16 (parameter table)
    if (p->dtype != ATTN_BF16 && p->dtype != ATTN_FP16) return ATTN_ERR_INVALID;
    if (p->d_rope != 0 || p->causal != 0 || p->dense_dq_mode != 0 || p->band != 0 || p->mask_align != 0 ||
        p->pre_tokens != 0 || p->next_tokens != 0)
      return ATTN_ERR_INVALID;
    // D is 192 or 128 (K and V may differ); N1, N2 in 1..128; G in 1..32
    if ((p->d_qk != 128 && p->d_qk != 192) || (p->d_v != 128 && p->d_v != 192)) return ATTN_ERR_INVALID;
    if (p->n1 > 128 || p->n2 > 128 || pl.G > 32) return ATTN_ERR_INVALID;
    // selectedBlockSize <= 128, multiple of 16; selectedBlockCount 1..128; count*size < 8K
    const int bs = p->block_size, cnt = p->block_count;
    if (bs <= 0 || bs > 128 || bs % 16) return ATTN_ERR_INVALID;
    if (cnt < 1 || cnt > 128 || (int64_t)cnt * bs >= 8192) return ATTN_ERR_INVALID;
    if (pl.T1 > kSelMaxT || pl.T2 > kSelMaxT) return ATTN_ERR_INVALID;
    pl.blkoff.assign(B + 1, 0);
    for (int b = 0; b < B; ++b) {
      const int64_t S1 = cq[b + 1] - cq[b], S2 = ck[b + 1] - ck[b];
      if (S1 > kSelMaxS || S2 > kSelMaxS) return ATTN_ERR_INVALID;
      // KV S of each sequence: a multiple of blockSize and >= count*size (read as >=)
      if (S2 % bs) return ATTN_ERR_INVALID;
      if (S1 > 0 && S2 < (int64_t)cnt * bs) return ATTN_ERR_INVALID;
      pl.blkoff[b + 1] = pl.blkoff[b] + (int32_t)(S2 / bs);
    }
    pl.nblk_total = pl.blkoff[B];
    if (!selected_supported(p->d_qk, p->d_v, pl.G, bs)) return ATTN_ERR_UNSUPPORTED;
    if (p->dkdv_atomic && !p->deterministic) return ATTN_ERR_UNSUPPORTED;
    pl.entries = pl.T1 * p->n2 * cnt;
    if (pl.entries >= (int64_t(1) << 31) || (int64_t)p->n2 * pl.nblk_total >= (int64_t(1) << 31))
      return ATTN_ERR_UNSUPPORTED;
    // Windows of query tokens: the backward's dQ shares of one window (cnt N1 d_qk elements per
    // token), or the forward's partials (cnt N1 (d_v elements + 8 bytes) per token), stay within
    // kSelShareMax; the caller may ask for smaller windows.  Windows are of equal length but
    // the last.
    if (p->sel_window_tokens < 0) return ATTN_ERR_INVALID;
    const uint64_t share_per_token = p->op == ATTN_OP_SELECTED_FWD ? (uint64_t)cnt * p->n1 * (p->d_v * 2 + 8)
                                                                   : (uint64_t)cnt * p->n1 * p->d_qk * 2;
    int64_t w = std::max<int64_t>(1, (int64_t)(kSelShareMax / share_per_token));
    if (p->sel_window_tokens > 0) w = std::min<int64_t>(w, p->sel_window_tokens);
    pl.nwin = (int)std::max<int64_t>(1, (pl.T1 + w - 1) / w);
    pl.win_tokens = std::max<int64_t>(1, (pl.T1 + pl.nwin - 1) / pl.nwin);
  }

  // ---- workspace layout ----
  size_t o = 0;
  pl.off_cu_q = o;  o += 8 * (size_t)(B + 1);
  pl.off_cu_kv = o; o += 8 * (size_t)(B + 1);
  pl.off_tab1 = o;
  if (p->op == ATTN_OP_DENSE) {
    o += 4 * pl.kv_tiles.size();
    pl.off_kvsplit = o;
    o += 4 * pl.kv_split.size();
    pl.off_tab2 = o;
    o += 4 * pl.q_tiles.size();
    pl.off_qt_base = o;
    o += 4 * pl.qt_base.size();
    pl.off_qt_kr = o;
    o += 4 * pl.qt_kr.size();
    o = (o + 7) / 8 * 8;
    pl.off_qt_blk = o;
    o += 8 * pl.qt_blk.size();
  } else {
    o += 4 * pl.blkoff.size();
    pl.off_tab2 = o;
  }
  pl.table_bytes = o;
  o = align_up(o);
  if (p->op == ATTN_OP_SELECTED_FWD) {  // the inverted index and the partials of one window
    const size_t nkeys = (size_t)p->n2 * pl.nblk_total;
    const size_t prow = (size_t)std::min<int64_t>(pl.win_tokens, pl.T1) * p->block_count * p->n1;  // (entry, head)
    pl.off_flag = o;    o = align_up(o + 4);
    pl.off_counts = o;  o = align_up(o + 4 * nkeys);
    pl.off_offsets = o; o = align_up(o + 4 * (nkeys + 1));
    pl.off_cursor = o;  o = align_up(o + 4 * nkeys);
    pl.off_list = o;    o = align_up(o + 4 * (size_t)pl.entries);
    pl.off_scratch = o; o = align_up(o + 8 * (size_t)pl.entries);
    pl.off_dq_part = o; o = align_up(o + 2 * prow * p->d_v);  // O_b / l_b
    pl.off_ml = o;      o = align_up(o + 8 * prow);           // (m_b, l_b)
    if (pl.nwin > 1) { pl.off_wofs = o; o = align_up(o + 4 * nkeys * (size_t)(pl.nwin + 1)); }
    pl.total = o;
    return ATTN_OK;
  }
  if (p->op == ATTN_OP_INDEXER) {
    const size_t nkeys = (size_t)p->n2 * pl.T2;
    pl.off_flag = o;  o = align_up(o + 4);
    pl.off_dkacc = o; o = align_up(o + 4 * nkeys * (size_t)p->d_qk);
    if (!pl.idx_atomic) {
      pl.off_counts = o;  o = align_up(o + 4 * nkeys);
      pl.off_offsets = o; o = align_up(o + 4 * (nkeys + 1));
      pl.off_cursor = o;  o = align_up(o + 4 * nkeys);
      pl.off_list = o;    o = align_up(o + 4 * (size_t)pl.entries);
      pl.off_scratch = o; o = align_up(o + 8 * (size_t)pl.entries);
      pl.off_contrib = o;
      o = align_up(o + 2 * (size_t)std::min<int64_t>(pl.win_tokens, pl.T1) * p->n2 * p->block_count * p->d_qk);
      if (pl.nwin > 1) { pl.off_wofs = o; o = align_up(o + 4 * nkeys * (size_t)(pl.nwin + 1)); }
    }
    pl.total = o;
    return ATTN_OK;
  }
  const size_t rows = (size_t)pl.T1 * p->n1;
  pl.off_lse2 = o; o = align_up(o + 4 * rows);
  pl.off_ndrow = o; o = align_up(o + 4 * rows);
  if (p->op == ATTN_OP_SELECTED) {
    const size_t nkeys = (size_t)p->n2 * pl.nblk_total;
    pl.off_counts = o;  o = align_up(o + 4 * nkeys);
    pl.off_offsets = o; o = align_up(o + 4 * (nkeys + 1));
    pl.off_cursor = o;  o = align_up(o + 4 * nkeys);
    pl.off_list = o;    o = align_up(o + 4 * (size_t)pl.entries);
    pl.off_scratch = o; o = align_up(o + 8 * (size_t)pl.entries);
    pl.off_flag = o;    o = align_up(o + 4);
    pl.off_dq_part = o;  // the shares of one window, then one (token, KV head) row group of scratch
    o = align_up(o + 2 * ((size_t)std::min<int64_t>(pl.win_tokens, pl.T1) * p->block_count * p->n1 + pl.G) * p->d_qk);
    if (pl.nwin > 1) {
      pl.off_wofs = o;  o = align_up(o + 4 * nkeys * (size_t)(pl.nwin + 1));
      pl.off_kvacc = o; o = align_up(o + 4 * nkeys * (size_t)sel_kv_keys(p->block_size) * (p->d_qk + p->d_v));
    }
  }
  if (p->op == ATTN_OP_DENSE && pl.dense_ds) {
    pl.off_ds = o;
    o = align_up(o + (size_t)pl.ds_blocks * p->n1 * kDenseTile * kDenseTile * 2);
  }
  if (p->op == ATTN_OP_DENSE && p->dtype == ATTN_BF16 && pl.kv_slots > 0) {
    pl.off_kvpart = o;
    o = align_up(o + (size_t)pl.kv_slots * kDenseKvPartBytes);
  }
  pl.total = o;
  return ATTN_OK;
}

// ---- pinned staging ring for the per-call tables --------------------------------
// The tables are written to a pinned host slot and copied into the workspace by the first
// kernel of the call (the row-statistics kernel reads the slot directly).  A slot is reused
// only after that kernel has executed (the event recorded behind it); the device's ring lock
// is held from choosing the slot until the event is recorded.
struct StagingSlot {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};
struct DeviceStaging {
  std::mutex mu;
  StagingSlot slots[4];
  int next = 0;
};
std::mutex g_staging_mu;
std::map<int, DeviceStaging*> g_staging;

class TableStage {
 public:
  ~TableStage() {
    if (lock_.owns_lock()) lock_.unlock();
  }
  // Copy bytes (zero-padded to a multiple of 16) into a free slot.
  hipError_t stage(const std::vector<uint8_t>& bytes) {
    if (bytes.empty()) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    DeviceStaging* ds;
    {
      std::lock_guard<std::mutex> lk(g_staging_mu);
      auto it = g_staging.find(dev);
      if (it == g_staging.end()) it = g_staging.emplace(dev, new DeviceStaging).first;
      ds = it->second;
    }
    lock_ = std::unique_lock<std::mutex>(ds->mu);
    StagingSlot& sl = ds->slots[ds->next];
    ds->next = (ds->next + 1) % 4;
    if (sl.pending) {
      e = hipEventSynchronize(sl.ev);
      if (e != hipSuccess) return e;
      sl.pending = false;
    }
    if (!sl.ev) {
      e = hipEventCreateWithFlags(&sl.ev, hipEventDisableTiming);
      if (e != hipSuccess) return e;
    }
    const size_t padded = (bytes.size() + 15) / 16 * 16;
    if (sl.cap < padded) {
      if (sl.host) (void)hipHostFree(sl.host);
      sl.host = nullptr;
      sl.cap = 0;
      const size_t cap = std::max<size_t>(padded, 4096);
      e = hipHostMalloc(&sl.host, cap, hipHostMallocDefault);
      if (e != hipSuccess) return e;
      sl.cap = cap;
    }
    std::memcpy(sl.host, bytes.data(), bytes.size());
    std::memset(static_cast<uint8_t*>(sl.host) + bytes.size(), 0, padded - bytes.size());
    slot_ = &sl;
    n16_ = (int64_t)(padded / 16);
    return hipSuccess;
  }
  const void* src() const { return slot_ ? slot_->host : nullptr; }
  int64_t n16() const { return n16_; }
  // After the launch of the kernel that reads the slot: the slot is busy until it has run.
  hipError_t commit(hipStream_t s) {
    if (!slot_) return hipSuccess;
    const hipError_t e = hipEventRecord(slot_->ev, s);
    if (e == hipSuccess) slot_->pending = true;
    lock_.unlock();
    return e;
  }

 private:
  std::unique_lock<std::mutex> lock_;
  StagingSlot* slot_ = nullptr;
  int64_t n16_ = 0;
};

std::vector<uint8_t> pack_tables(const attn_bwd_problem_t* p, const Plan& pl) {
  std::vector<uint8_t> t(pl.table_bytes, 0);
  std::memcpy(t.data() + pl.off_cu_q, pl.cuq.data(), 8 * (size_t)(pl.B + 1));
  std::memcpy(t.data() + pl.off_cu_kv, pl.cukv.data(), 8 * (size_t)(pl.B + 1));
  if (p->op == ATTN_OP_DENSE) {
    if (!pl.kv_tiles.empty()) std::memcpy(t.data() + pl.off_tab1, pl.kv_tiles.data(), 4 * pl.kv_tiles.size());
    if (!pl.kv_split.empty()) std::memcpy(t.data() + pl.off_kvsplit, pl.kv_split.data(), 4 * pl.kv_split.size());
    if (!pl.q_tiles.empty()) std::memcpy(t.data() + pl.off_tab2, pl.q_tiles.data(), 4 * pl.q_tiles.size());
    std::memcpy(t.data() + pl.off_qt_base, pl.qt_base.data(), 4 * pl.qt_base.size());
    if (!pl.qt_kr.empty()) std::memcpy(t.data() + pl.off_qt_kr, pl.qt_kr.data(), 4 * pl.qt_kr.size());
    if (!pl.qt_blk.empty()) std::memcpy(t.data() + pl.off_qt_blk, pl.qt_blk.data(), 8 * pl.qt_blk.size());
  } else {
    std::memcpy(t.data() + pl.off_tab1, pl.blkoff.data(), 4 * pl.blkoff.size());
  }
  return t;
}

// ---- optional per-kernel timing (attn_bwd_profiling) ------------------------------
struct ProfRec { const char* name; hipEvent_t a, b; };
struct ProfTotal { const char* name; double ms; int64_t n; };
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<ProfRec> g_prof_pending;
std::vector<ProfTotal> g_prof_totals;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Run one launcher; while profiling is on, bracket it with events on the stream.
template <typename F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return launch();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    a = prof_event();
    b = prof_event();
  }
  if (!a || !b) return launch();
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = launch();
  const hipError_t e2 = hipEventRecord(b, s);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_pending.push_back({name, a, b});
  return e != hipSuccess ? e : e2;
}

bool misaligned(const void* ptr) { return ptr && (reinterpret_cast<uintptr_t>(ptr) & 15u); }

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off); }

// Pointer checks of the dense call (after validate_and_plan).
attn_status_t dense_check_pointers(const attn_bwd_problem_t* p, const Plan& pl, const void* q, const void* q_rope,
                                   const void* k, const void* k_rope, const void* v, const void* out, const void* dy,
                                   const float* softmax_max, const float* softmax_sum, void* dq, void* dq_rope,
                                   void* dk, void* dk_rope, void* dv) {
  if (p->op != ATTN_OP_DENSE) return ATTN_ERR_INVALID;
  const bool has_q = pl.T1 > 0, has_k = pl.T2 > 0;
  if (has_q && (!q || !out || !dy || !softmax_max || !softmax_sum || !dq)) return ATTN_ERR_NULLPTR;
  if (has_k && (!k || !v || !dk || !dv)) return ATTN_ERR_NULLPTR;
  if (p->d_rope > 0) {
    if ((has_q && (!q_rope || !dq_rope)) || (has_k && (!k_rope || !dk_rope))) return ATTN_ERR_NULLPTR;
  } else if (q_rope || k_rope || dq_rope || dk_rope) {
    return ATTN_ERR_INVALID;
  }
  for (const void* ptr : {q, q_rope, k, k_rope, v, out, dy, (const void*)softmax_max, (const void*)softmax_sum,
                          (const void*)dq, (const void*)dq_rope, (const void*)dk, (const void*)dk_rope, (const void*)dv})
    if (misaligned(ptr)) return ATTN_ERR_INVALID;
  return ATTN_OK;
}

// Enqueue the dense backward with `workspace` (pl.total bytes, 256-byte aligned).  no_alloc: the
// tables are copied with hipMemcpyAsync from pageable host memory (the pinned staging ring
// allocates on first use) and the per-kernel timing, which creates events, is bypassed.
attn_status_t dense_launch(const attn_bwd_problem_t* p, const Plan& pl, const void* q, const void* q_rope,
                           const void* k, const void* k_rope, const void* v, const void* out, const void* dy,
                           const float* softmax_max, const float* softmax_sum, void* dq, void* dq_rope, void* dk,
                           void* dk_rope, void* dv, void* workspace, hipStream_t s, bool no_alloc) {
  if (pl.T1 == 0 && pl.T2 == 0) return ATTN_OK;
  auto run = [&](const char* name, auto&& launch) -> hipError_t { return no_alloc ? launch() : timed(name, s, launch); };
  TableStage tables;
  const std::vector<uint8_t> tab = pack_tables(p, pl);
  if (no_alloc) {
    // pageable source: the copy has taken the bytes when the call returns
    if (!tab.empty() && hipMemcpyAsync(workspace, tab.data(), tab.size(), hipMemcpyHostToDevice, s) != hipSuccess)
      return ATTN_ERR_HIP;
  } else if (tables.stage(tab) != hipSuccess) {
    return ATTN_ERR_HIP;
  }

  PreArgs pa{};
  pa.out = out; pa.dy = dy; pa.smax = softmax_max; pa.ssum = softmax_sum;
  pa.lse2 = at<float>(workspace, pl.off_lse2); pa.ndrow = at<float>(workspace, pl.off_ndrow);
  pa.rows = pl.T1 * p->n1; pa.dv = p->d_v; pa.elem = p->dtype == ATTN_BF16 ? 0 : 2;
  pa.tab_src = static_cast<const uint4*>(tables.src()); pa.tab_dst = static_cast<uint4*>(workspace);
  pa.tab_n16 = no_alloc ? 0 : tables.n16();
  if (run("row_stats", [&] { return launch_preprocess(pa, s); }) != hipSuccess) return ATTN_ERR_HIP;
  if (!no_alloc && tables.commit(s) != hipSuccess) return ATTN_ERR_HIP;

  DenseArgs a{};
  a.q = q; a.q_rope = q_rope; a.k = k; a.k_rope = k_rope; a.v = v; a.dy = dy;
  a.lse2 = pa.lse2; a.ndrow = pa.ndrow;
  a.dq = dq; a.dq_rope = dq_rope; a.dk = dk; a.dk_rope = dk_rope; a.dv = dv;
  a.cu_q = at<const int64_t>(workspace, pl.off_cu_q);
  a.cu_kv = at<const int64_t>(workspace, pl.off_cu_kv);
  a.kv_tiles = at<const int32_t>(workspace, pl.off_tab1);
  a.q_tiles = at<const int32_t>(workspace, pl.off_tab2);
  a.qt_base = at<const int32_t>(workspace, pl.off_qt_base);
  a.qt_kr = at<const int32_t>(workspace, pl.off_qt_kr);
  a.qt_blk = at<const int64_t>(workspace, pl.off_qt_blk);
  a.ds = pl.dense_ds ? at<void>(workspace, pl.off_ds) : nullptr;
  a.kv_split = at<const int32_t>(workspace, pl.off_kvsplit);
  a.kv_part = pl.kv_slots > 0 ? at<void>(workspace, pl.off_kvpart) : nullptr;
  a.n_kv_tiles = (int)(pl.kv_tiles.size() / 6);
  a.n_kv_split = (int)(pl.kv_split.size() / 5);
  a.n_q_tiles = (int)(pl.q_tiles.size() / 2);
  a.batch = pl.B; a.n1 = p->n1; a.n2 = p->n2; a.G = pl.G;
  a.T1 = pl.T1; a.T2 = pl.T2;
  a.d_main = p->d_qk; a.d_rope = p->d_rope; a.d_v = p->d_v;
  a.scale = (float)p->scale;
  a.scale_log2e = (float)(p->scale * 1.4426950408889634);
  a.mask_on = p->causal || p->band;
  a.lo_rel = pl.lo_rel; a.hi_rel = pl.hi_rel; a.align = p->mask_align;
  if (p->dtype == ATTN_FP32)
    return run("dense_fp32", [&] { return launch_dense_fp32(a, s); }) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
  if (run("dense_kv_major", [&] { return launch_dense_kv_bf16(a, s); }) != hipSuccess) return ATTN_ERR_HIP;
  if (pl.dense_ds) {
    // one launch: the split key tiles' dK / dV, then dQ = dS K
    if (run("dense_dq", [&] { return launch_dense_dq_from_ds(a, s); }) != hipSuccess) return ATTN_ERR_HIP;
  } else {
    if (a.n_kv_split > 0 && run("dense_kv_combine", [&] { return launch_dense_kv_combine(a, s); }) != hipSuccess)
      return ATTN_ERR_HIP;
    if (run("dense_dq_recompute", [&] { return launch_dense_dq_bf16(a, s); }) != hipSuccess) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

// ---- fixed scratch for attn_bwd_dense_varlen_noalloc --------------------------------------
// Device memory beyond the inputs and outputs for callers that cannot allocate: one array per
// GPU, held from module load to process end.  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, once per device (with that
// device current), and is kept here.
constexpr size_t kNoAllocScratch = ATTN_BWD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratch];
std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & (kAlign - 1))) return hipErrorInvalidValue;
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* attn_bwd_status_string(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULLPTR: return "null pointer";
    case ATTN_ERR_INVALID: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported combination";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* attn_bwd_version(void) { return "0.1.0"; }

attn_status_t attn_bwd_workspace_size(const attn_bwd_problem_t* p, uint64_t* bytes) {
  if (!bytes) return ATTN_ERR_NULLPTR;
  Plan pl;
  const attn_status_t st = validate_and_plan(p, pl);
  if (st != ATTN_OK) return st;
  *bytes = pl.total;
  return ATTN_OK;
}

attn_status_t attn_bwd_dense_varlen(const attn_bwd_problem_t* p, const void* q, const void* q_rope,
                                    const void* k, const void* k_rope, const void* v, const void* out,
                                    const void* dy, const float* softmax_max, const float* softmax_sum,
                                    void* dq, void* dq_rope, void* dk, void* dk_rope, void* dv,
                                    void* workspace, uint64_t workspace_bytes, void* hip_stream) {
  Plan pl;
  attn_status_t st = validate_and_plan(p, pl);
  if (st != ATTN_OK) return st;
  st = dense_check_pointers(p, pl, q, q_rope, k, k_rope, v, out, dy, softmax_max, softmax_sum, dq, dq_rope, dk,
                            dk_rope, dv);
  if (st != ATTN_OK) return st;
  if (!workspace || workspace_bytes < pl.total || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return ATTN_ERR_WORKSPACE;
  return dense_launch(p, pl, q, q_rope, k, k_rope, v, out, dy, softmax_max, softmax_sum, dq, dq_rope, dk, dk_rope,
                      dv, workspace, static_cast<hipStream_t>(hip_stream), false);
}

attn_status_t attn_bwd_dense_varlen_noalloc(const attn_bwd_problem_t* p, const void* q, const void* q_rope,
                                            const void* k, const void* k_rope, const void* v, const void* out,
                                            const void* dy, const float* softmax_max, const float* softmax_sum,
                                            void* dq, void* dq_rope, void* dk, void* dk_rope, void* dv,
                                            void* hip_stream) {
  Plan pl;
  attn_status_t st = validate_and_plan(p, pl);
  if (st != ATTN_OK) return st;
  // dQ mode 0 (automatic): stored dS when its plan fits the scratch array, else recomputation
  attn_bwd_problem_t q2;
  if (p->op == ATTN_OP_DENSE && p->dtype == ATTN_BF16 && p->dense_dq_mode == 0 && pl.total > kNoAllocScratch) {
    q2 = *p;
    q2.dense_dq_mode = 2;
    p = &q2;
    pl = Plan();
    st = validate_and_plan(p, pl);
    if (st != ATTN_OK) return st;
  }
  st = dense_check_pointers(p, pl, q, q_rope, k, k_rope, v, out, dy, softmax_max, softmax_sum, dq, dq_rope, dk,
                            dk_rope, dv);
  if (st != ATTN_OK) return st;
  if (pl.total > kNoAllocScratch) return ATTN_ERR_WORKSPACE;
  void* scratch_ptr = nullptr;
  if (noalloc_scratch(&scratch_ptr) != hipSuccess) return ATTN_ERR_HIP;
  return dense_launch(p, pl, q, q_rope, k, k_rope, v, out, dy, softmax_max, softmax_sum, dq, dq_rope, dk, dk_rope,
                      dv, scratch_ptr, static_cast<hipStream_t>(hip_stream), true);
}

attn_status_t attn_bwd_selected(const attn_bwd_problem_t* p, const void* q, const void* k, const void* v,
                                const void* out, const void* dy, const float* softmax_max,
                                const float* softmax_sum, const int32_t* topk_indices, void* dq, void* dk,
                                void* dv, void* workspace, uint64_t workspace_bytes, void* hip_stream) {
  Plan pl;
  attn_status_t st = validate_and_plan(p, pl);
  if (st != ATTN_OK) return st;
  if (p->op != ATTN_OP_SELECTED) return ATTN_ERR_INVALID;
  const bool has_q = pl.T1 > 0, has_k = pl.T2 > 0;
  // attentionOut is optional (parameter table): without it rowsum(P * dP) is formed from the
  // gathered rows by a KV-major pass instead of rowsum(dY * O)
  if (has_q && (!q || !dy || !softmax_max || !softmax_sum || !topk_indices || !dq)) return ATTN_ERR_NULLPTR;
  if (has_k && (!k || !v || !dk || !dv)) return ATTN_ERR_NULLPTR;
  for (const void* ptr : {q, k, v, out, dy, (const void*)softmax_max, (const void*)softmax_sum,
                          (const void*)topk_indices, (const void*)dq, (const void*)dk, (const void*)dv})
    if (misaligned(ptr)) return ATTN_ERR_INVALID;
  if (!workspace || workspace_bytes < pl.total || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return ATTN_ERR_WORKSPACE;
  if (!has_q && !has_k) return ATTN_OK;

  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  TableStage tables;
  if (tables.stage(pack_tables(p, pl)) != hipSuccess) return ATTN_ERR_HIP;

  PreArgs pa{};
  pa.out = out; pa.dy = dy; pa.smax = softmax_max; pa.ssum = softmax_sum;
  pa.lse2 = at<float>(workspace, pl.off_lse2); pa.ndrow = at<float>(workspace, pl.off_ndrow);
  pa.rows = pl.T1 * p->n1; pa.dv = p->d_v; pa.elem = p->dtype == ATTN_FP16 ? 1 : 0;
  pa.tab_src = static_cast<const uint4*>(tables.src()); pa.tab_dst = static_cast<uint4*>(workspace);
  pa.tab_n16 = tables.n16();
  if (timed("row_stats", s, [&] { return launch_preprocess(pa, s); }) != hipSuccess) return ATTN_ERR_HIP;
  if (tables.commit(s) != hipSuccess) return ATTN_ERR_HIP;
  SelArgs a{};
  a.q = q; a.k = k; a.v = v; a.dy = dy; a.lse2 = pa.lse2; a.ndrow = pa.ndrow; a.topk = topk_indices;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.cu_q = at<const int64_t>(workspace, pl.off_cu_q);
  a.cu_kv = at<const int64_t>(workspace, pl.off_cu_kv);
  a.blkoff = at<const int32_t>(workspace, pl.off_tab1);
  a.batch = pl.B; a.n1 = p->n1; a.n2 = p->n2; a.G = pl.G;
  a.d_qk = p->d_qk; a.d_v = p->d_v; a.bs = p->block_size; a.cnt = p->block_count;
  a.nblk_total = pl.nblk_total; a.T1 = pl.T1; a.T2 = pl.T2;
  a.scale = (float)p->scale;
  a.scale_log2e = (float)(p->scale * 1.4426950408889634);
  a.counts = at<int32_t>(workspace, pl.off_counts);
  a.offsets = at<int32_t>(workspace, pl.off_offsets);
  a.cursor = at<int32_t>(workspace, pl.off_cursor);
  a.list = at<int32_t>(workspace, pl.off_list);
  a.sort_scratch = at<int32_t>(workspace, pl.off_scratch);
  a.flag = at<int32_t>(workspace, pl.off_flag);
  a.dq_part = at<void>(workspace, pl.off_dq_part);
  a.nwin = pl.nwin;
  a.win_tokens = pl.win_tokens;
  a.wofs = pl.nwin > 1 ? at<int32_t>(workspace, pl.off_wofs) : nullptr;
  a.kvacc = pl.nwin > 1 ? at<float>(workspace, pl.off_kvacc) : nullptr;
  a.is_f16 = p->dtype == ATTN_FP16;
  if (timed("selected_index", s, [&] {
        const hipError_t e = launch_selected_index(a, s);
        return e != hipSuccess ? e : launch_selected_window_offsets(a, s);
      }) != hipSuccess)
    return ATTN_ERR_HIP;
  if (!out && has_q) {
    // rowsum(P dP) over the gathered rows, KV-major over the same index and windows; the
    // per-entry sums use the share buffer before the backward's first window does
    SelFwdArgs f{};
    f.q = q; f.k = k; f.v = v; f.dy = dy; f.topk = topk_indices;
    f.cu_q = a.cu_q; f.cu_kv = a.cu_kv;
    f.lse2 = pa.lse2; f.ndrow = pa.ndrow;
    f.batch = pl.B; f.n1 = p->n1; f.n2 = p->n2; f.G = pl.G; f.d_qk = p->d_qk; f.d_v = p->d_v;
    f.bs = p->block_size; f.cnt = p->block_count; f.T1 = pl.T1;
    f.scale_log2e = a.scale_log2e;
    f.is_f16 = a.is_f16;
    f.blkoff = a.blkoff; f.offsets = a.offsets; f.list = a.list; f.sched = a.cursor; f.wofs = a.wofs;
    f.nblk_total = pl.nblk_total; f.nwin = pl.nwin;
    f.part_d = static_cast<float*>(a.dq_part);
    for (int w = 0; w < pl.nwin; ++w) {
      f.win = w;
      f.t0 = std::min<int64_t>(pl.T1, (int64_t)w * pl.win_tokens);
      f.t1 = std::min<int64_t>(pl.T1, f.t0 + pl.win_tokens);
      if (timed("selected_row_stat", s, [&] {
            const hipError_t e = launch_selected_drow_kv(f, s);
            return e != hipSuccess ? e : launch_selected_drow_combine(f, s);
          }) != hipSuccess)
        return ATTN_ERR_HIP;
    }
  }
  for (int w = 0; w < pl.nwin; ++w) {
    a.win = w;
    a.t0 = std::min<int64_t>(pl.T1, (int64_t)w * pl.win_tokens);
    a.t1 = std::min<int64_t>(pl.T1, a.t0 + pl.win_tokens);
    if (timed("selected_kv_major", s, [&] { return launch_selected_kv(a, s); }) != hipSuccess) return ATTN_ERR_HIP;
    if (timed("selected_dq_reduce", s, [&] { return launch_selected_dq_reduce(a, s); }) != hipSuccess)
      return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

attn_status_t attn_fwd_selected(const attn_bwd_problem_t* p, const void* q, const void* k, const void* v,
                                const int32_t* topk_indices, void* out, float* softmax_max, float* softmax_sum,
                                void* workspace, uint64_t workspace_bytes, void* hip_stream) {
  Plan pl;
  attn_status_t st = validate_and_plan(p, pl);
  if (st != ATTN_OK) return st;
  if (p->op != ATTN_OP_SELECTED_FWD) return ATTN_ERR_INVALID;
  const bool has_q = pl.T1 > 0;
  if (has_q && (!q || !k || !v || !topk_indices || !out || !softmax_max || !softmax_sum)) return ATTN_ERR_NULLPTR;
  for (const void* ptr : {q, k, v, (const void*)topk_indices, (const void*)out, (const void*)softmax_max,
                          (const void*)softmax_sum})
    if (misaligned(ptr)) return ATTN_ERR_INVALID;
  if (!workspace || workspace_bytes < pl.total || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return ATTN_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  int32_t* flag = at<int32_t>(workspace, pl.off_flag);
  if (launch_fill_i32(flag, 1, 0, s) != hipSuccess) return ATTN_ERR_HIP;
  if (!has_q) return ATTN_OK;
  TableStage tables;
  if (tables.stage(pack_tables(p, pl)) != hipSuccess) return ATTN_ERR_HIP;
  PreArgs pa{};  // no rows: the launch only copies the tables into the workspace
  pa.tab_src = static_cast<const uint4*>(tables.src()); pa.tab_dst = static_cast<uint4*>(workspace);
  pa.tab_n16 = tables.n16();
  if (timed("tables", s, [&] { return launch_preprocess(pa, s); }) != hipSuccess) return ATTN_ERR_HIP;
  if (tables.commit(s) != hipSuccess) return ATTN_ERR_HIP;
  // the inverted index of the ids: the KV-major pass walks each block's list
  SelArgs x{};
  x.topk = topk_indices;
  x.cu_q = at<const int64_t>(workspace, pl.off_cu_q);
  x.blkoff = at<const int32_t>(workspace, pl.off_tab1);
  x.batch = pl.B; x.n2 = p->n2; x.cnt = p->block_count; x.nblk_total = pl.nblk_total; x.T1 = pl.T1;
  x.counts = at<int32_t>(workspace, pl.off_counts);
  x.offsets = at<int32_t>(workspace, pl.off_offsets);
  x.cursor = at<int32_t>(workspace, pl.off_cursor);
  x.list = at<int32_t>(workspace, pl.off_list);
  x.sort_scratch = at<int32_t>(workspace, pl.off_scratch);
  x.flag = flag;
  x.nwin = pl.nwin; x.win_tokens = pl.win_tokens;
  x.wofs = pl.nwin > 1 ? at<int32_t>(workspace, pl.off_wofs) : nullptr;
  if (timed("selected_index", s, [&] {
        const hipError_t e = launch_selected_index(x, s);
        return e != hipSuccess ? e : launch_selected_window_offsets(x, s);
      }) != hipSuccess)
    return ATTN_ERR_HIP;
  SelFwdArgs f{};
  f.q = q; f.k = k; f.v = v; f.topk = topk_indices;
  f.cu_q = x.cu_q;
  f.cu_kv = at<const int64_t>(workspace, pl.off_cu_kv);
  f.o = out; f.smax = softmax_max; f.ssum = softmax_sum; f.flag = flag;
  f.batch = pl.B; f.n1 = p->n1; f.n2 = p->n2; f.G = pl.G; f.d_qk = p->d_qk; f.d_v = p->d_v;
  f.bs = p->block_size; f.cnt = p->block_count; f.T1 = pl.T1;
  f.scale_log2e = (float)(p->scale * 1.4426950408889634);
  f.is_f16 = p->dtype == ATTN_FP16;
  f.blkoff = x.blkoff; f.offsets = x.offsets; f.list = x.list; f.sched = x.cursor; f.wofs = x.wofs;
  f.nblk_total = pl.nblk_total; f.nwin = pl.nwin;
  f.part_o = at<void>(workspace, pl.off_dq_part);
  f.part_ml = at<float2>(workspace, pl.off_ml);
  for (int w = 0; w < pl.nwin; ++w) {
    f.win = w;
    f.t0 = std::min<int64_t>(pl.T1, (int64_t)w * pl.win_tokens);
    f.t1 = std::min<int64_t>(pl.T1, f.t0 + pl.win_tokens);
    if (timed("selected_forward", s, [&] { return launch_selected_forward_kv(f, s); }) != hipSuccess)
      return ATTN_ERR_HIP;
    if (timed("selected_forward_combine", s, [&] { return launch_selected_forward_combine(f, s); }) != hipSuccess)
      return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

attn_status_t attn_bwd_selected_index(const attn_bwd_problem_t* p, const int32_t* topk_indices, int32_t* offsets,
                                      int32_t* lists, int32_t* order, void* workspace, uint64_t workspace_bytes,
                                      void* hip_stream) {
  Plan pl;
  attn_status_t st = validate_and_plan(p, pl);
  if (st != ATTN_OK) return st;
  if (p->op != ATTN_OP_SELECTED) return ATTN_ERR_INVALID;
  if (!offsets || !order || (pl.entries > 0 && (!topk_indices || !lists))) return ATTN_ERR_NULLPTR;
  if (!workspace || workspace_bytes < pl.total || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return ATTN_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  TableStage tables;
  if (tables.stage(pack_tables(p, pl)) != hipSuccess) return ATTN_ERR_HIP;
  PreArgs pa{};  // no rows: the launch only copies the tables into the workspace
  pa.tab_src = static_cast<const uint4*>(tables.src()); pa.tab_dst = static_cast<uint4*>(workspace);
  pa.tab_n16 = tables.n16();
  if (launch_preprocess(pa, s) != hipSuccess) return ATTN_ERR_HIP;
  if (tables.commit(s) != hipSuccess) return ATTN_ERR_HIP;
  SelArgs a{};
  a.topk = topk_indices;
  a.cu_q = at<const int64_t>(workspace, pl.off_cu_q);
  a.blkoff = at<const int32_t>(workspace, pl.off_tab1);
  a.batch = pl.B; a.n2 = p->n2; a.cnt = p->block_count; a.nblk_total = pl.nblk_total; a.T1 = pl.T1;
  a.counts = at<int32_t>(workspace, pl.off_counts);
  a.offsets = at<int32_t>(workspace, pl.off_offsets);
  a.cursor = at<int32_t>(workspace, pl.off_cursor);
  a.list = at<int32_t>(workspace, pl.off_list);
  a.sort_scratch = at<int32_t>(workspace, pl.off_scratch);
  a.flag = at<int32_t>(workspace, pl.off_flag);
  if (launch_selected_index(a, s) != hipSuccess) return ATTN_ERR_HIP;
  const size_t nkeys = (size_t)p->n2 * pl.nblk_total;
  if (hipMemcpyAsync(offsets, a.offsets, 4 * (nkeys + 1), hipMemcpyDeviceToDevice, s) != hipSuccess ||
      hipMemcpyAsync(order, a.cursor, 4 * nkeys, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return ATTN_ERR_HIP;
  if (pl.entries > 0 && hipMemcpyAsync(lists, a.list, 4 * (size_t)pl.entries, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status_t attn_bwd_indexer(const attn_bwd_problem_t* p, const void* q, const void* k, const void* weights,
                               const void* dy, const int32_t* indices, void* dq, void* dk, void* dweights,
                               void* workspace, uint64_t workspace_bytes, void* hip_stream) {
  Plan pl;
  attn_status_t st = validate_and_plan(p, pl);
  if (st != ATTN_OK) return st;
  if (p->op != ATTN_OP_INDEXER) return ATTN_ERR_INVALID;
  const bool has_q = pl.T1 > 0, has_k = pl.T2 > 0;
  if (has_q && (!q || !weights || !dy || !indices || !dq || !dweights)) return ATTN_ERR_NULLPTR;
  if (has_k && (!k || !dk)) return ATTN_ERR_NULLPTR;
  for (const void* ptr : {q, k, (const void*)dq, (const void*)dk}) if (misaligned(ptr)) return ATTN_ERR_INVALID;
  for (const void* ptr : {weights, dy, (const void*)dweights, (const void*)indices})  // 2- and 4-byte elements
    if (ptr && (reinterpret_cast<uintptr_t>(ptr) & 3u)) return ATTN_ERR_INVALID;
  if (!workspace || workspace_bytes < pl.total || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return ATTN_ERR_WORKSPACE;
  if (!has_q && !has_k) return ATTN_OK;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  TableStage tables;
  if (tables.stage(pack_tables(p, pl)) != hipSuccess) return ATTN_ERR_HIP;
  PreArgs pa{};  // no rows: the launch only copies the tables into the workspace
  pa.tab_src = static_cast<const uint4*>(tables.src()); pa.tab_dst = static_cast<uint4*>(workspace);
  pa.tab_n16 = tables.n16();
  if (timed("tables", s, [&] { return launch_preprocess(pa, s); }) != hipSuccess) return ATTN_ERR_HIP;
  if (tables.commit(s) != hipSuccess) return ATTN_ERR_HIP;
  IdxArgs a{};
  a.q = q; a.k = k; a.weights = weights; a.dy = dy; a.indices = indices;
  a.dq = dq; a.dk = dk; a.dweights = dweights;
  a.dk_acc = at<float>(workspace, pl.off_dkacc);
  a.cu_q = at<const int64_t>(workspace, pl.off_cu_q);
  a.cu_kv = at<const int64_t>(workspace, pl.off_cu_kv);
  a.flag = at<int32_t>(workspace, pl.off_flag);
  a.batch = pl.B; a.n1 = p->n1; a.n2 = p->n2; a.G = pl.G; a.d = p->d_qk; a.topk = p->block_count;
  a.T1 = pl.T1; a.T2 = pl.T2;
  a.atomic = pl.idx_atomic;
  a.nkeys = (int64_t)p->n2 * pl.T2;
  if (launch_fill_i32(a.flag, 1, 0, s) != hipSuccess) return ATTN_ERR_HIP;
  if (timed("indexer_zero", s, [&] { return launch_indexer_zero(a, s); }) != hipSuccess) return ATTN_ERR_HIP;
  if (a.atomic) {
    a.unit0 = 0;
    a.unit1 = pl.T1 * p->n2;
    if (timed("indexer_query_major", s, [&] { return launch_indexer_qm(a, s); }) != hipSuccess) return ATTN_ERR_HIP;
  } else {
    // the inverted index of the indices (one key per index) for the ordered dK sums
    SelArgs x{};
    x.topk = indices; x.cu_q = a.cu_q; x.blkoff = at<const int32_t>(workspace, pl.off_tab1);
    x.batch = pl.B; x.n2 = p->n2; x.cnt = p->block_count; x.nblk_total = pl.nblk_total; x.T1 = pl.T1;
    x.counts = at<int32_t>(workspace, pl.off_counts);
    x.offsets = at<int32_t>(workspace, pl.off_offsets);
    x.cursor = at<int32_t>(workspace, pl.off_cursor);
    x.list = at<int32_t>(workspace, pl.off_list);
    x.sort_scratch = at<int32_t>(workspace, pl.off_scratch);
    x.flag = a.flag;
    x.nwin = pl.nwin; x.win_tokens = pl.win_tokens;
    x.wofs = pl.nwin > 1 ? at<int32_t>(workspace, pl.off_wofs) : nullptr;
    if (timed("indexer_index", s, [&] {
          const hipError_t e = launch_selected_index(x, s);
          return e != hipSuccess ? e : launch_selected_window_offsets(x, s);
        }) != hipSuccess)
      return ATTN_ERR_HIP;
    a.offsets = x.offsets; a.list = x.list; a.wofs = x.wofs; a.nwin = pl.nwin;
    a.contrib = at<uint16_t>(workspace, pl.off_contrib);
    for (int w = 0; w < pl.nwin; ++w) {
      a.win = w;
      const int64_t t0 = std::min<int64_t>(pl.T1, (int64_t)w * pl.win_tokens);
      const int64_t t1 = std::min<int64_t>(pl.T1, t0 + pl.win_tokens);
      a.unit0 = t0 * p->n2;
      a.unit1 = t1 * p->n2;
      if (timed("indexer_query_major", s, [&] { return launch_indexer_qm(a, s); }) != hipSuccess) return ATTN_ERR_HIP;
      if (timed("indexer_dk_reduce", s, [&] { return launch_indexer_dk_reduce(a, s); }) != hipSuccess)
        return ATTN_ERR_HIP;
    }
  }
  return timed("indexer_dk_cast", s, [&] { return launch_indexer_dk_cast(a, s); }) == hipSuccess ? ATTN_OK
                                                                                                  : ATTN_ERR_HIP;
}

attn_status_t attn_bwd_check_index_flag(const attn_bwd_problem_t* p, const void* workspace, int32_t* raised,
                                        void* hip_stream) {
  if (!raised || !workspace) return ATTN_ERR_NULLPTR;
  Plan pl;
  attn_status_t st = validate_and_plan(p, pl);
  if (st != ATTN_OK) return st;
  if (p->op == ATTN_OP_DENSE) return ATTN_ERR_INVALID;
  int32_t h = 0;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (hipMemcpyAsync(&h, static_cast<const uint8_t*>(workspace) + pl.off_flag, 4, hipMemcpyDeviceToHost, s) !=
          hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return ATTN_ERR_HIP;
  *raised = h ? 1 : 0;
  return ATTN_OK;
}

attn_status_t attn_bwd_profiling(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on.store(enable != 0, std::memory_order_relaxed);
  return ATTN_OK;
}

attn_status_t attn_bwd_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof_pending) {
    (void)hipEventSynchronize(r.b);
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_pending.clear();
  g_prof_totals.clear();
  return ATTN_OK;
}

attn_status_t attn_bwd_profile_read(int32_t index, const char** name, double* total_ms, int64_t* launches) {
  if (!name || !total_ms || !launches) return ATTN_ERR_NULLPTR;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return ATTN_ERR_HIP;
    auto it = std::find_if(g_prof_totals.begin(), g_prof_totals.end(),
                           [&](const ProfTotal& t) { return std::strcmp(t.name, r.name) == 0; });
    if (it == g_prof_totals.end()) g_prof_totals.push_back({r.name, (double)ms, 1});
    else { it->ms += ms; it->n += 1; }
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_pending.clear();
  if (index < 0 || index >= (int32_t)g_prof_totals.size()) return ATTN_ERR_INVALID;
  *name = g_prof_totals[index].name;
  *total_ms = g_prof_totals[index].ms;
  *launches = g_prof_totals[index].n;
  return ATTN_OK;
}

}  // extern "C"
