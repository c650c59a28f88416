// Inverted index of topkIndices for the KV-major selected backward.
//
// Page "NsaSelectedAttentionGrad", formula section: selectedKey = Gather(key, topkIndices[i]);
// the gradient of a gather is a scatter-add (page "aclnnLightningIndexerGrad", formula:
// dK = ScatterAdd(..., Indices)).  Instead of scattering with atomics, the index is
// inverted so that each (KV head, block) -- a key -- owns the list of its entries
// t * cnt + slot in ascending order.  Keys are numbered kv_head * nblk_total + blkoff[b] + id.
// An id outside [0, S2_b / block_size) is skipped (and raises the flag).
//
// Ordered path (a stable counting sort; used when the per-chunk count table fits the
// scratch buffer and a key histogram fits in LDS):
//   1. hist:    the entries are cut into chunks of consecutive entries; each chunk's key
//               histogram (LDS) becomes one row of a [chunk][key] table
//   2. column sum:  per key, the sum over chunks -> counts
//   3. scan:        exclusive prefix sum of the counts -> offsets
//   4. column scan: per key, offsets + running sum over chunks -> each (chunk, key) base
//   5. fill:    one wave walks its chunk in entry order; an entry's position is its key's
//               running base plus its rank among equal keys of the same 64 entries
// Entry order is ascending t * cnt + slot within a key, so no sort is needed.
// Fallback path: atomic count, scan, atomic fill, then an LDS / global bitonic sort of each
// key's segment.  Both give the same lists.
// Schedule: the keys in classes of list length, each class about 4/5 as long as the one before
// it -- with thresholds t_0 = the longest length, t_(k+1) = floor(4 t_k / 5), class k holds the
// lengths in (t_(k+1), t_k], 32 classes, the last also holding every shorter list -- longest
// class first, and in key order within a class.  The workgroups with the longest lists start
// first (the late ones are short, as in longest-first order), and those running at the same
// time mostly belong to one KV head (and, for varlen batches, one sequence): lists drawn from
// one distribution whose spread is below a fifth of the longest fall into one class.  Such
// workgroups gather the same query rows -- a token's Q/dY rows for one KV head are read by
// every block it chose -- and when those blocks run together the repeated reads are served
// from the caches instead of HBM.
// Identity order (which is head-major too) when there are too many keys.
// Integer work only: bitwise reproducible.
#include <algorithm>
#include <climits>

#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

constexpr int kSortCap = 16384;  // segments up to this length are sorted in LDS
constexpr int kMaxLdsKeys = 16384;  // ordered path: key histogram in LDS (64 KiB)
constexpr int kMaxChunks = 2048;
constexpr int kSchedCap = 8192;     // keys sorted for the schedule in LDS (8 bytes each, 64 KiB)

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

// entry e = (t n2 + kvh) cnt + slot with topk value id
__device__ __forceinline__ bool decode_id(const SelArgs& a, int64_t e, int id, int64_t& t, int& slot, int& key) {
  slot = (int)(e % a.cnt);
  const int64_t tn = e / a.cnt;
  const int kvh = (int)(tn % a.n2);
  t = tn / a.n2;
  const int b = seq_of(a.cu_q, a.batch, t);
  const int nblk = a.blkoff[b + 1] - a.blkoff[b];
  if (id < 0 || id >= nblk) return false;
  key = kvh * a.nblk_total + a.blkoff[b] + id;
  return true;
}

__device__ __forceinline__ bool decode_entry(const SelArgs& a, int64_t e, int64_t& t, int& slot, int& key) {
  return decode_id(a, e, a.topk[e], t, slot, key);
}

__global__ __launch_bounds__(256) void idx_count_kernel(SelArgs a, int64_t total) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  int64_t t; int slot, key;
  if (decode_entry(a, e, t, slot, key)) atomicAdd(&a.counts[key], 1);
  else a.flag[0] = 1;
}

__global__ __launch_bounds__(256) void idx_fill_kernel(SelArgs a, int64_t total) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  int64_t t; int slot, key;
  if (decode_entry(a, e, t, slot, key)) {
    const int pos = atomicAdd(&a.cursor[key], 1);
    a.list[pos] = (int32_t)(t * a.cnt + slot);
  }
}

// Single-workgroup exclusive scan: offsets[i] = sum counts[0..i), offsets[n] = total.
__global__ __launch_bounds__(1024) void idx_scan_kernel(const int32_t* counts, int32_t* offsets, int32_t* cursor, int n) {
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int32_t carry = 0;
  for (int base = 0; base < n; base += 4096) {
    int32_t v[4], tsum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = base + tid * 4 + k;
      v[k] = idx < n ? counts[idx] : 0;
      tsum += v[k];
    }
    int32_t x = tsum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    if (wid == 0) {
      int32_t ws = lane < 16 ? wsum[lane] : 0;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const int32_t y = __shfl_up(ws, off);
        if (lane >= off) ws += y;
      }
      if (lane < 16) wsum[lane] = ws;
    }
    __syncthreads();
    int32_t run = carry + (wid > 0 ? wsum[wid - 1] : 0) + (x - tsum);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = base + tid * 4 + k;
      if (idx < n) { offsets[idx] = run; cursor[idx] = run; }
      run += v[k];
    }
    const int32_t total = wsum[15];
    __syncthreads();
    carry += total;
  }
  if (tid == 0) offsets[n] = carry;
}

template <typename Buf>
__device__ void bitonic_sort(Buf s, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const int32_t x = s[i], y = s[ixj];
          const bool up = (i & k) == 0;
          if ((x > y) == up) { s[i] = y; s[ixj] = x; }
        }
      }
      __threadfence_block();
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(256) void idx_sort_kernel(const int32_t* offsets, int32_t* list, int32_t* scratch) {
  __shared__ int32_t s[kSortCap];
  const int key = blockIdx.x;
  const int o0 = offsets[key];
  const int len = offsets[key + 1] - o0;
  if (len <= 1) return;
  int n = 1;
  while (n < len) n <<= 1;
  if (n <= kSortCap) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) s[i] = i < len ? list[o0 + i] : INT_MAX;
    __syncthreads();
    bitonic_sort(s, n);
    for (int i = threadIdx.x; i < len; i += blockDim.x) list[o0 + i] = s[i];
  } else {
    // Long segment: sort in global memory, in this key's private region of the scratch
    // buffer ([2*o0, 2*o0 + n) with n < 2*len, disjoint from every other key's region).
    int32_t* buf = scratch + 2 * (int64_t)o0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) buf[i] = i < len ? list[o0 + i] : INT_MAX;
    __threadfence_block();
    __syncthreads();
    bitonic_sort(buf, n);
    for (int i = threadIdx.x; i < len; i += blockDim.x) list[o0 + i] = buf[i];
  }
}

// ---- ordered path -------------------------------------------------------------------------

__global__ __launch_bounds__(256) void idx_hist_kernel(SelArgs a, int64_t total, int64_t chunk, int nkeys,
                                                       int32_t* tab) {
  extern __shared__ int32_t hist[];
  for (int k = threadIdx.x; k < nkeys; k += 256) hist[k] = 0;
  __syncthreads();
  const int64_t e0 = (int64_t)blockIdx.x * chunk, e1 = min(total, e0 + chunk);
  for (int64_t e = e0 + threadIdx.x; e < e1; e += 256) {
    int64_t t; int slot, key;
    if (decode_entry(a, e, t, slot, key)) atomicAdd(&hist[key], 1);
    else a.flag[0] = 1;
  }
  __syncthreads();
  int32_t* row = tab + (int64_t)blockIdx.x * nkeys;
  for (int k = threadIdx.x; k < nkeys; k += 256) row[k] = hist[k];
}

// Column pass over the [chunk][key] table: a workgroup takes 16 keys, and each of its 64
// chunk lanes a contiguous range of at most 32 chunks (nchunks <= 2048).  SCAN = false:
// counts[key] = sum over all chunks.  SCAN = true: every entry becomes offsets[key] plus the
// sum of the entries of the earlier chunks (in place).
template <bool SCAN>
__global__ __launch_bounds__(1024) void idx_colpass_kernel(int32_t* tab, int nchunks, int nkeys, int32_t* counts,
                                                           const int32_t* offsets) {
  __shared__ int32_t part[64][16];
  const int kq = threadIdx.x & 15, cl = threadIdx.x >> 4;
  const int key = blockIdx.x * 16 + kq;
  const bool kok = key < nkeys;
  const int cpl = (nchunks + 63) / 64;
  const int c0 = min(nchunks, cl * cpl), c1 = min(nchunks, c0 + cpl);
  int32_t sum = 0;
  if (kok)
    for (int c = c0; c < c1; ++c) sum += tab[(int64_t)c * nkeys + key];
  part[cl][kq] = sum;
  __syncthreads();
  int32_t before = 0;
  for (int j = 0; j < cl; ++j) before += part[j][kq];
  if (!kok) return;
  if constexpr (!SCAN) {
    if (cl == 63) counts[key] = before + sum;
  } else {
    int32_t run = offsets[key] + before;
    for (int c = c0; c < c1; ++c) {
      const int64_t i = (int64_t)c * nkeys + key;
      const int32_t v = tab[i];
      tab[i] = run;
      run += v;
    }
  }
}

// One wave per chunk.  Per round of 64 consecutive entries: rank = number of lower lanes
// with the same key; the highest lane of each key advances that key's base.  The lanes of
// one key are found bit by bit (one ballot per key bit); the next round's ids are loaded
// while a round is placed.
__global__ __launch_bounds__(64) void idx_fill_ordered_kernel(SelArgs a, int64_t total, int64_t chunk, int nkeys,
                                                              const int32_t* tab) {
  extern __shared__ int32_t base[];
  const int lane = threadIdx.x;
  const int32_t* row = tab + (int64_t)blockIdx.x * nkeys;
  for (int k = lane; k < nkeys; k += 64) base[k] = row[k];
  __syncthreads();
  const int kbits = nkeys > 1 ? 32 - __builtin_clz(nkeys - 1) : 0;
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  const int64_t e0 = (int64_t)blockIdx.x * chunk, e1 = min(total, e0 + chunk);
  int id_next = e0 + lane < e1 ? a.topk[e0 + lane] : -1;
  for (int64_t r0 = e0; r0 < e1; r0 += 64) {
    const int64_t e = r0 + lane;
    const int id = id_next;
    id_next = e + 64 < e1 ? a.topk[e + 64] : -1;
    int64_t t = 0; int slot = 0, key = -1;
    if (e >= e1 || !decode_id(a, e, id, t, slot, key)) key = -1;
    uint64_t same = __ballot(key >= 0);
    for (int bit = 0; bit < kbits; ++bit) {
      const bool one = (key >> bit) & 1;
      const uint64_t bb = __ballot(one);
      same &= one ? bb : ~bb;
    }
    const int rank = __popcll(same & below);
    const bool last = (same >> lane) <= 1;  // no higher lane holds the key
    int pos = 0;
    if (key >= 0) pos = base[key] + rank;
    __syncthreads();  // every lane has read its base before any is advanced
    if (key >= 0) {
      a.list[pos] = (int32_t)(t * a.cnt + slot);
      if (last) base[key] = pos + 1;
    }
    __syncthreads();
  }
}

// Schedule: keys by length class, longest class first; key order within a class.  One
// workgroup.
constexpr int kSchedClasses = 32;
__device__ int length_class(int len, int longest) {
  int t = longest;
  for (int k = 0; k < kSchedClasses - 1; ++k) {
    t = (int)((int64_t)t * 4 / 5);
    if (len > t) return k;
  }
  return kSchedClasses - 1;
}
__global__ __launch_bounds__(1024) void idx_schedule_kernel(const int32_t* offsets, int nkeys, int32_t* sched) {
  extern __shared__ uint64_t sk[];
  __shared__ int longest;
  if (threadIdx.x == 0) longest = 0;
  __syncthreads();
  int mx = 0;
  for (int i = threadIdx.x; i < nkeys; i += 1024) mx = max(mx, offsets[i + 1] - offsets[i]);
  atomicMax(&longest, mx);
  __syncthreads();
  int n = 1;
  while (n < nkeys) n <<= 1;
  for (int i = threadIdx.x; i < n; i += 1024) {
    // ascending order of (class, key); class 0 holds the longest lists
    sk[i] = i < nkeys ? ((uint64_t)length_class(offsets[i + 1] - offsets[i], longest) << 32) | (uint32_t)i : ~0ull;
  }
  __syncthreads();
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += 1024) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = sk[i], y = sk[ixj];
          const bool up = (i & k) == 0;
          if ((x > y) == up) { sk[i] = y; sk[ixj] = x; }
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < nkeys; i += 1024) sched[i] = (int32_t)(uint32_t)sk[i];
}

__global__ __launch_bounds__(256) void idx_identity_kernel(int32_t* sched, int nkeys) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k < nkeys) sched[k] = k;
}

// Window offsets: for every key and window boundary w (0..nwin), the first position of the
// key's list whose entry t cnt + slot has t >= w win_tokens (lists are ascending), found by
// binary search.  wofs[key][0] = offsets[key], wofs[key][nwin] = offsets[key + 1].
__global__ __launch_bounds__(256) void idx_window_kernel(const int32_t* offsets, const int32_t* list, int32_t* wofs,
                                                         int nkeys, int nwin, int64_t win_tokens, int64_t T1,
                                                         int cnt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)nkeys * (nwin + 1)) return;
  const int key = (int)(i / (nwin + 1)), w = (int)(i - (int64_t)key * (nwin + 1));
  int lo = offsets[key], hi = offsets[key + 1];
  if (w == nwin) {
    wofs[i] = hi;
    return;
  }
  const int64_t target = min((int64_t)w * win_tokens, T1) * cnt;  // first entry of window w
  while (lo < hi) {  // first position with list[pos] >= target
    const int mid = lo + ((hi - lo) >> 1);
    if ((int64_t)list[mid] < target) lo = mid + 1;
    else hi = mid;
  }
  wofs[i] = lo;
}

unsigned grid_for(int64_t n, int64_t per_block) {
  int64_t b = (n + per_block - 1) / per_block;
  return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_selected_window_offsets(const SelArgs& a, hipStream_t s) {
  const int nkeys = a.n2 * a.nblk_total;
  if (a.nwin <= 1 || nkeys == 0) return hipSuccess;
  const int64_t n = (int64_t)nkeys * (a.nwin + 1);
  hipLaunchKernelGGL(idx_window_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, (const int32_t*)a.offsets,
                     (const int32_t*)a.list, a.wofs, nkeys, a.nwin, a.win_tokens, a.T1, a.cnt);
  return hipGetLastError();
}

// Chunking of the ordered path: at most kMaxChunks chunks of a multiple of 64 entries,
// and a count table no larger than the 2 * entries ints of the sort scratch buffer.
// Returns 0 chunks when the ordered path does not apply.
static void ordered_plan(int64_t total, int nkeys, int& nchunks, int64_t& chunk) {
  nchunks = 0;
  chunk = 0;
  if (total <= 0 || nkeys <= 0 || nkeys > kMaxLdsKeys) return;
  int64_t n = (total + 1023) / 1024;
  n = std::min<int64_t>(n, kMaxChunks);
  n = std::min<int64_t>(n, 2 * total / nkeys);
  if (n < 1) return;
  chunk = ((total + n - 1) / n + 63) / 64 * 64;
  nchunks = (int)((total + chunk - 1) / chunk);
}

hipError_t launch_selected_index(const SelArgs& a, hipStream_t s) {
  const int nkeys = a.n2 * a.nblk_total;
  const int64_t total = a.T1 * a.n2 * a.cnt;
  hipError_t e = launch_fill_i32(a.flag, 1, 0, s);
  if (e != hipSuccess) return e;
  if (nkeys == 0) return hipSuccess;
  int nchunks;
  int64_t chunk;
  ordered_plan(total, nkeys, nchunks, chunk);
  const unsigned kgrid = grid_for(nkeys, 256);
  if (nchunks > 0) {
    int32_t* tab = a.sort_scratch;
    const size_t lds = 4 * (size_t)nkeys;
    hipLaunchKernelGGL(idx_hist_kernel, dim3(nchunks), dim3(256), lds, s, a, total, chunk, nkeys, tab);
    const dim3 cgrid((unsigned)((nkeys + 15) / 16));
    hipLaunchKernelGGL(idx_colpass_kernel<false>, cgrid, dim3(1024), 0, s, tab, nchunks, nkeys, a.counts,
                       (const int32_t*)nullptr);
    hipLaunchKernelGGL(idx_scan_kernel, dim3(1), dim3(1024), 0, s, (const int32_t*)a.counts, a.offsets, a.cursor, nkeys);
    hipLaunchKernelGGL(idx_colpass_kernel<true>, cgrid, dim3(1024), 0, s, tab, nchunks, nkeys, (int32_t*)nullptr,
                       (const int32_t*)a.offsets);
    hipLaunchKernelGGL(idx_fill_ordered_kernel, dim3(nchunks), dim3(64), lds, s, a, total, chunk, nkeys,
                       (const int32_t*)tab);
  } else {
    e = launch_fill_i32(a.counts, nkeys, 0, s);
    if (e != hipSuccess) return e;
    if (total > 0) hipLaunchKernelGGL(idx_count_kernel, dim3(grid_for(total, 256)), dim3(256), 0, s, a, total);
    hipLaunchKernelGGL(idx_scan_kernel, dim3(1), dim3(1024), 0, s, (const int32_t*)a.counts, a.offsets, a.cursor, nkeys);
    if (total > 0) {
      hipLaunchKernelGGL(idx_fill_kernel, dim3(grid_for(total, 256)), dim3(256), 0, s, a, total);
      hipLaunchKernelGGL(idx_sort_kernel, dim3((unsigned)nkeys), dim3(256), 0, s, (const int32_t*)a.offsets, a.list,
                         a.sort_scratch);
    }
  }
  // the schedule reuses the cursor array (the fill above is done with it)
  if (nkeys <= kSchedCap)
    hipLaunchKernelGGL(idx_schedule_kernel, dim3(1), dim3(1024), 8 * (size_t)(nkeys <= 1 ? 1 : 1 << (32 - __builtin_clz(nkeys - 1))),
                       s, (const int32_t*)a.offsets, nkeys, a.cursor);
  else
    hipLaunchKernelGGL(idx_identity_kernel, dim3(kgrid), dim3(256), 0, s, a.cursor, nkeys);
  return hipGetLastError();
}

}  // namespace ab
