// dn_tfrag.h -- workspace layout of the per-chunk T = (I + A)^{-1} diag(beta)
// matrices, shared by the kernel that writes them (WY prep) and the one that
// reads them (state scan).
//
// T is lower triangular.  Row tile t (16 rows) owns the 32-column blocks
// kb = 0 .. t/2 of the lower triangle; block (t, kb) is stored as two planes
// (hi, lo) of 64 lanes x 16 bytes, lane (g = lane / 16, i = lane % 16) holding
//   T[16 t + i][32 kb + 4 g .. + 3]       (bytes 0..7: 16x16 tile (t, 2 kb))
//   T[16 t + i][32 kb + 16 + 4 g .. + 3]  (bytes 8..15: tile (t, 2 kb + 1))
// as bf16 -- an A operand of a 16x16x32 bf16 MFMA whose contraction slot
// (g, e) stands for column 32 kb + 4 g + e (e < 4) or 32 kb + 16 + 4 g + e - 4
// (e >= 4), so the consumer loads it straight into registers.  Tiles above
// the diagonal are stored as zeros.  Blocks are numbered row tile by row
// tile: tile t starts at block base(t).
#pragma once

#include <stddef.h>

namespace dn {

template <int C>
struct Frag {
  static constexpr int NT = C / 16;
  __host__ __device__ static constexpr int base(int t) {
    return (t & 1) ? (t / 2 + 1) * (t / 2 + 1) : (t / 2) * (t / 2 + 1);
  }
  static constexpr int NBLK = base(NT);
  static constexpr size_t chunk_u4 = (size_t)NBLK * 2 * 64;  // uint4 per chunk
};

}  // namespace dn
