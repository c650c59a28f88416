"""Host check of the selected dQ-share chunk layout (csrc/share_layout.hpp): for every head
count G up to 64 and both query widths, share_chunk must be a bijection of the G x DQK/8 chunks
of a share and share_pos its inverse, and with G a multiple or a divisor of 16 each 16-row
MFMA tile's (16 rows x 4 chunks) store must land on contiguous chunks.  Compiled with g++."""
import os
import shutil
import subprocess

import pytest

HDR = os.path.join(os.path.dirname(__file__), "..", "sparse_attention_backward_amd", "csrc", "share_layout.hpp")

PROG = r"""
#include <cstdio>
#include <vector>
#include "share_layout.hpp"
using namespace ab;
template <int DQK> int check() {
  int bad = 0;
  for (int G = 1; G <= 64; ++G) {
    const int R = share_rows(G), n = G * DQK / 8;
    std::vector<int> seen(n, 0);
    for (int h = 0; h < G; ++h)
      for (int k = 0; k < DQK / 8; ++k) {
        const int c = share_chunk<DQK>(h, k, R);
        if (c < 0 || c >= n) { ++bad; continue; }
        ++seen[c];
        if (share_pos<DQK>(c, R) != h * (DQK / 8) + k) ++bad;
      }
    for (int i = 0; i < n; ++i) bad += seen[i] != 1;
    if (G % 16 == 0 || 16 % G == 0) {
      // one store: rows r0 .. r0 + 15 of the step (heads r % G), chunks 4 q .. 4 q + 3
      for (int r0 = 0; r0 < 64; r0 += 16)
        for (int q = 0; q < DQK / 32; ++q) {
          const int e = G >= 16 ? 1 : 16 / G;  // shares touched by the tile
          for (int s = 0; s < e; ++s) {
            int lo = 1 << 30, hi = -1;
            for (int l = 0; l < 16; ++l) {
              if (G < 16 && l / G != s) continue;
              for (int g = 0; g < 4; ++g) {
                const int c = share_chunk<DQK>((r0 + l) % G, 4 * q + g, R);
                lo = c < lo ? c : lo; hi = c > hi ? c : hi;
              }
            }
            const int rows = G < 16 ? G : 16;
            if (hi - lo + 1 != 4 * rows) ++bad;
          }
        }
    }
  }
  return bad;
}
int main() { std::printf("%d %d\n", check<192>(), check<128>()); return 0; }
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_share_layout_is_a_permutation_with_contiguous_tile_stores(tmp_path):
    src = tmp_path / "t.cpp"
    src.write_text(PROG)
    exe = tmp_path / "t"
    subprocess.run(["g++", "-std=c++17", "-O1", "-D__host__=", "-D__device__=", "-I", os.path.dirname(HDR),
                    str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    assert out == ["0", "0"]
