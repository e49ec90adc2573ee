// dn_ktile.h -- LDS layout of a chunk's k tile, shared by the WY-prep and
// state-scan kernels.
//
// The tile is C rows x d_k bf16, row-major, with the 16-byte chunks of each
// row XOR-swizzled by a function of the row.  The swizzle keeps the two
// access patterns the kernels use free of LDS bank conflicts:
//   * 16-byte row reads (an MFMA operand: lanes i = 0..15 read rows r0 + i,
//     lane group g reads 16-byte chunk 4 kb + g);
//   * 8-byte transposing reads of K^T (ds_read_b64_tr_b16: lanes 4 m + a of a
//     16-lane group read row r0 + m, columns 16 dt + 4 a .. + 3).
#pragma once

namespace dn {

template <int DK>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (DK == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return ((row >> 2) & 3) | ((row & 2) << 1);
}

// Element offset of 16-byte chunk `ch` (elements 8 ch .. 8 ch + 7) of row `row`.
template <int DK>
__device__ __forceinline__ int koff(int row, int ch) {
  return row * DK + ((ch ^ kswz<DK>(row)) << 3);
}

}  // namespace dn
