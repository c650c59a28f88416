// Inverted index of topkIndices for the KV-major selected backward.
//
// Page "NsaSelectedAttentionGrad", formula section: selectedKey = Gather(key, topkIndices[i]);
// the gradient of a gather is a scatter-add (page "aclnnLightningIndexerGrad", formula:
// dK = ScatterAdd(..., Indices)).  Instead of scattering with atomics, the index is
// inverted so that each (KV head, block) owns the list of query tokens that selected it:
//   1. count:  histogram of entries per key = (kv head, sequence block)      (int atomics)
//   2. scan:   exclusive prefix sum of the counts -> offsets
//   3. fill:   each entry e = (t, kv head, slot) writes t * cnt + slot at a claimed position
//   4. sort:   each key's segment is sorted ascending, which removes the arbitrary order of
//              step 3: the lists, and every sum taken over them, are deterministic.
// Keys are numbered kv_head * nblk_total + blkoff[b] + id.  An id outside
// [0, S2_b / block_size) is skipped (and raises the flag); steps 1 and 3 skip the same
// entries, so the offsets and the filled lists agree.
// Integer work only: bitwise reproducible.
#include <climits>

#include "common.hpp"
#include "kernels.hpp"

namespace ab {

namespace {

constexpr int kSortCap = 16384;  // segments up to this length are sorted in LDS

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

__device__ __forceinline__ bool decode_entry(const SelArgs& a, int64_t e, int64_t& t, int& slot, int& key) {
  slot = (int)(e % a.cnt);
  const int64_t tn = e / a.cnt;
  const int kvh = (int)(tn % a.n2);
  t = tn / a.n2;
  const int b = seq_of(a.cu_q, a.batch, t);
  const int nblk = a.blkoff[b + 1] - a.blkoff[b];
  const int id = a.topk[e];
  if (id < 0 || id >= nblk) return false;
  key = kvh * a.nblk_total + a.blkoff[b] + id;
  return true;
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

hipError_t launch_selected_index(const SelArgs& a, hipStream_t s) {
  const int nkeys = a.n2 * a.nblk_total;
  const int64_t total = a.T1 * a.n2 * a.cnt;
  hipError_t e = launch_fill_i32(a.flag, 1, 0, s);
  if (e != hipSuccess) return e;
  e = launch_fill_i32(a.counts, nkeys, 0, s);
  if (e != hipSuccess) return e;
  if (nkeys == 0) return hipSuccess;
  if (total > 0) hipLaunchKernelGGL(idx_count_kernel, dim3(grid_for(total, 256)), dim3(256), 0, s, a, total);
  hipLaunchKernelGGL(idx_scan_kernel, dim3(1), dim3(1024), 0, s, (const int32_t*)a.counts, a.offsets, a.cursor, nkeys);
  if (total > 0) {
    hipLaunchKernelGGL(idx_fill_kernel, dim3(grid_for(total, 256)), dim3(256), 0, s, a, total);
    hipLaunchKernelGGL(idx_sort_kernel, dim3((unsigned)nkeys), dim3(256), 0, s, (const int32_t*)a.offsets, a.list,
                       a.sort_scratch);
  }
  return hipGetLastError();
}

}  // namespace ab
