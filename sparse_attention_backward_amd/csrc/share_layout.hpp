// Layout of the selected backward's dQ shares, shared by the KV-major kernel that writes them
// and the reduction that reads them.
#pragma once

namespace ab {

// Layout of a selected dQ share (the G x DQK values one (token, slot, KV head) contributes)
// in 16-byte chunks of 8 consecutive features: the chunk of head h, row chunk k sits at
//   (h / R) R (DQK / 8) + k R + h % R,   R = share_rows(G),
// i.e. blocks of R heads, chunk-major inside a block.  When 16-row MFMA tiles hold whole
// blocks (R = min(G, 16) for G a multiple or a divisor of 16) the 16 rows x 4 chunks that one
// store instruction of the KV-major kernel writes are contiguous; otherwise R = 1, plain
// row-major order.  share_pos inverts it: the chunk's place in the G x DQK row-major block.
__host__ __device__ constexpr int share_rows(int G) {
  return (G % 16 == 0 || 16 % G == 0) ? (G < 16 ? G : 16) : 1;
}
template <int DQK>
__host__ __device__ constexpr int share_chunk(int h, int k, int R) {
  return (h / R) * R * (DQK / 8) + k * R + h % R;
}
template <int DQK>
__host__ __device__ constexpr int share_pos(int c, int R) {
  const int blk = c / (R * (DQK / 8)), rem = c - blk * R * (DQK / 8);
  return (blk * R + rem % R) * (DQK / 8) + rem / R;
}

}  // namespace ab
