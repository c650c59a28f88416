// Shared device helpers for the gfx950 attention-backward kernels.
//
// MFMA lane layouts used throughout (64-lane wavefront, l = lane id, g = l / 16):
//   v_mfma_f32_16x16x32_bf16   A (16 x 32): lane holds row l%16, k = 8g .. 8g+7
//                              B (32 x 16): lane holds col l%16, k = 8g .. 8g+7
//                              C (16 x 16): lane holds col l%16, rows 4g .. 4g+3
//   v_mfma_f32_16x16x16_bf16   A / B as above with k = 4g .. 4g+3, same C.
// A contraction may permute its k index freely as long as A and B agree, so the
// C tile of one product (lane: fixed column, four consecutive rows) feeds the A
// operand of the next product when two row tiles are packed into the 8 k-slots:
// slot j < 4 <- rows 4g+j of tile t0, slot j >= 4 <- rows 4g+j-4 of tile t1.
//
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, output lane i,
// element j comes from element i%4 of the 8-byte word addressed by lane 4j + i/4
// of the same group.  If lane (jj = (l%16)/4, q = l%4) addresses
// &M[row(jj)][c0 + 4q] of a row-major bf16 tile M, lane i of the group receives
// M[row(j)][c0 + i] for j = 0..3: a column slice, i.e. the B operand of an MFMA
// whose k index runs over rows of M.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ab {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) f16x8 lds_f16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Transposed 4 x bf16 read from LDS (see header comment).  `p` points into LDS.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Reads at an LDS byte address (an integer); a constant added to the address becomes the
// instruction's immediate offset.
__device__ __forceinline__ bf16x8 lds_b128_at(uint32_t addr) {
  return *reinterpret_cast<const lds_bf16x8*>((uintptr_t)addr);
}
__device__ __forceinline__ f16x8 lds_f16x8_at(uint32_t addr) {
  return *reinterpret_cast<const lds_f16x8*>((uintptr_t)addr);
}
__device__ __forceinline__ f32x4 lds_f32x4_at(uint32_t addr) {
  return *reinterpret_cast<const lds_f32x4*>((uintptr_t)addr);
}
__device__ __forceinline__ float lds_f32_at(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) float*>((uintptr_t)addr);
}
__device__ __forceinline__ i16x4 lds_tr16_at(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4*>((uintptr_t)addr));
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
__device__ __forceinline__ void lds_st16_at(uint32_t addr, uint4 v) {
  *reinterpret_cast<lds_u32x4*>((uintptr_t)addr) = u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ void lds_st4_at(uint32_t addr, float v) {
  *reinterpret_cast<__attribute__((address_space(3))) float*>((uintptr_t)addr) = v;
}
// Hides how a value was computed, so that the compiler keeps it as one base register and
// folds the constants added to it into immediate offsets instead of re-associating the
// sum into one register per constant.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm("" : "+v"(x));
  return x;
}

__device__ __forceinline__ bf16x8 join8(i16x4 lo, i16x4 hi) {
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);  // round to nearest even
}

// Pack eight floats (two C tiles' four values each) into an A operand.
__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
  bf16x8 r;
  r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
  r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
  return r;
}

__device__ __forceinline__ i16x4 pack4(f32x4 v) {
  bf16x4 r;
  r[0] = (__bf16)v[0]; r[1] = (__bf16)v[1]; r[2] = (__bf16)v[2]; r[3] = (__bf16)v[3];
  return __builtin_bit_cast(i16x4, r);
}

// ---- element types: bf16 and fp16 operands of the 16x16x32 MFMA, fp32 accumulation ----
template <typename T>
struct Mma;
template <>
struct Mma<__bf16> {
  typedef bf16x8 v8;
  static __device__ __forceinline__ f32x4 run(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mma<_Float16> {
  typedef f16x8 v8;
  static __device__ __forceinline__ f32x4 run(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <typename T, typename X>
__device__ __forceinline__ typename Mma<T>::v8 as_v8(X x) {
  return __builtin_bit_cast(typename Mma<T>::v8, x);
}
// Eight floats (two C tiles' four values each) as one operand, round to nearest even.
template <typename T>
__device__ __forceinline__ typename Mma<T>::v8 pack8t(f32x4 lo, f32x4 hi) {
  typename Mma<T>::v8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (T)lo[i];
    r[4 + i] = (T)hi[i];
  }
  return r;
}
// float -> the 16-bit pattern of T (round to nearest even), and back
template <typename T>
__device__ __forceinline__ uint16_t f2t(float f) {
  return __builtin_bit_cast(uint16_t, (T)f);
}
template <typename T>
__device__ __forceinline__ float t2f(uint16_t x) {
  return (float)__builtin_bit_cast(T, x);
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ void sts16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Non-temporal 16-byte accesses, for data read or written once (not worth keeping in the caches).
__device__ __forceinline__ uint4 ldg16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void sts16_stream(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// LDS tile of bf16 rows, C columns, no padding.  The 16-byte chunk c of row r is stored at
// chunk c ^ h(r), with h the RowTile swizzle below (2 (r & 7), or 2 ((r >> 1) & 3) for rows
// of 32 (mod 64) words): a ds_read_b128 over 16 consecutive rows at one column chunk and a
// ds_read_b64_tr_b16 over 8 consecutive rows x 32 contiguous bytes run at the LDS's linear
// rate (measured; see RowTile).
template <int C>
struct Swz {
  static_assert(C % 64 == 0, "swizzled rows hold a multiple of 64 bf16");
  static constexpr int W = C / 2;
  static_assert(W % 64 == 32 || (W % 64 == 0 && C % 128 == 0), "unsupported row length");
  __device__ __forceinline__ static int h(int r) {
    if constexpr (W % 64 == 32) return 2 * ((r >> 1) & 3);
    else return 2 * (r & 7);
  }
  // element offset of (row r, column col); columns col..col+k stay contiguous while
  // they lie in one 8-element chunk
  __device__ __forceinline__ static int off(int r, int col) { return r * C + (((col >> 3) ^ h(r)) << 3) + (col & 7); }
  // h touches the low HB bits of a chunk index only
  static constexpr int HB = (W % 64 == 32) ? 3 : 4, M = 1 << HB;
};

// Addresses of the chunks STEP*k + part (k unrolled at compile time, part per lane) of
// rows that share h: the XOR only changes the low HB bits, so the offset is a per-lane
// table of M/STEP entries plus a compile-time multiple of M chunks.  Keeps swizzled
// addressing to a few registers instead of one per access.
template <int C, int STEP>
struct SwzCursor {
  static constexpr int M = Swz<C>::M, T = M / STEP;
  static_assert(M % STEP == 0, "step must divide the swizzle period");
  int lo[T];
  __device__ __forceinline__ void init(int r, int part) {
    const int hh = Swz<C>::h(r);
#pragma unroll
    for (int t = 0; t < T; ++t) lo[t] = ((STEP * t + part) ^ hh) << 3;
  }
  // element offset of chunk STEP*k + part within its row
  __device__ __forceinline__ int off(int k) const { return (k / T) * (M * 8) + lo[k % T]; }
};

// LDS tile of 64 rows of W 16-byte chunks (W = 8 or 16), row-major, filled by
// global->LDS transfers that each move 1024 contiguous LDS bytes = RPI = 64 / W whole rows
// (lane l: row l / W, slot l % W).  Chunk c of row r sits in slot c ^ swz(r); the lane that
// fills a slot reads the matching chunk, so every transfer reads whole rows (full cache
// lines).  swz(r) = 2 (r & 7) for 256-byte rows and 2 ((r >> 1) & 3) for 128-byte rows
// (the XOR never touches chunk bit 0).  Measured on gfx950 (LDS cycles per instruction,
// rocprofv3 SQ_LDS_IDX_ACTIVE / SQ_INSTS_LDS, with the operand offsets below):
//   * the A-operand ds_read_b128 (16 rows at one chunk per lane group) takes 4 cycles, the
//     rate of a linear 1 KiB read; folding row bit 3 into chunk bit 0 as well makes it
//     2-way bank conflicted (8 cycles);
//   * the transposed ds_read_b64_tr_b16 of colB (8 rows x 32 contiguous bytes) takes 2
//     cycles, the rate of a linear 512-byte read;
//   * colK, four chunks of a row at one 8-byte half per lane, is 2-way conflicted (4
//     cycles) whatever the XOR, unless the rows with bit 1 of swz set keep their chunk
//     halves swapped (2 cycles).
template <int W>
struct RowTile {
  static_assert(W == 8 || W == 16, "rows of 128 or 256 bytes");
  static constexpr int RB = 16 * W;        // bytes per row
  static constexpr int RPI = 1024 / RB;    // rows per transfer instruction
  static constexpr int BYTES = 64 * RB;
  __host__ __device__ static constexpr int swz(int r) {
    if constexpr (W == 16) return 2 * (r & 7);
    else return 2 * ((r >> 1) & 3);
  }
  __host__ __device__ static constexpr int off(int r, int c) { return r * RB + 16 * (c ^ swz(r)); }

  // Per-lane offsets of the MFMA operand reads (l16 = lane & 15, g = lane >> 4):
  //   rowA(lane, s): A operand rows l16 at chunk 4s + g (16-byte reads; +16 RB for row tile 1);
  //   colB(lane, j): transposed B operand, rows 4g + l16/4 at chunk 2j + (l16&3)/2, half l16&1
  //                  (8-byte reads; +16 RB for the second 16 rows);
  //   colK(lane, m): the same rows at chunk 4m + (l16&3) (a B operand whose four 4-column
  //                  pieces are chunks 4m .. 4m + 3).
  // swz only XORs the chunk index with a value of the row, so the reads of k-step s, column
  // group j or chunk group m differ from those of 0 in bits 5-7 alone: rowA(l, s) =
  // rowA(l, 0) ^ 64 s, colB(l, j) = colB(l, 0) ^ 32 j, colK(l, m) = colK(l, 0) ^ 64 m (checked
  // by xor_steps).  Bits 0-7 of a 256-byte aligned base are zero, so base + rowA(l, s) =
  // (base + rowA(l, 0)) ^ 64 s: one address per part and stage and one XOR per fragment,
  // with the row offsets in the instruction's offset field.
  __host__ __device__ static constexpr int rowA(int lane, int s) { return off(lane & 15, 4 * s + (lane >> 4)); }
  __host__ __device__ static constexpr int colB(int lane, int j) {
    return off(4 * (lane >> 4) + ((lane & 15) >> 2), 2 * j + ((lane & 3) >> 1)) + 8 * (lane & 1);
  }
  __host__ __device__ static constexpr int colK(int lane, int m) {
    return off(4 * (lane >> 4) + ((lane & 15) >> 2), 4 * m + (lane & 3));
  }
  static constexpr bool xor_steps() {
    for (int lane = 0; lane < 64; ++lane) {
      if (rowA(lane, 0) >= 16 * RB || colB(lane, 0) >= 16 * RB || colK(lane, 0) >= 16 * RB) return false;
      for (int s = 0; s < W / 4; ++s)
        if (rowA(lane, s) != (rowA(lane, 0) ^ (64 * s)) || colK(lane, s) != (colK(lane, 0) ^ (64 * s))) return false;
      for (int j = 0; j < W / 2; ++j)
        if (colB(lane, j) != (colB(lane, 0) ^ (32 * j))) return false;
    }
    return true;
  }
};
static_assert(RowTile<8>::xor_steps() && RowTile<16>::xor_steps(), "operand offsets differ by XOR constants");

// Sequence of a packed row: largest b with cu[b] <= row (cu has B + 1 entries).
__device__ __forceinline__ int seq_of(const int64_t* cu, int batch, int64_t row) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int seq_of32(const int32_t* cu, int batch, int32_t v) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= v) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace ab
