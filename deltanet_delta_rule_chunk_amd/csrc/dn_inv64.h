// dn_inv64.h -- X = (I + A)^{-1} for a strictly lower-triangular 64 x 64
// fp32 matrix A in LDS, on the first four waves of a workgroup, for the
// 64-row-chunk matrix-core prep of the per-dimension decay.
//
// By 16 x 16 blocks, with D_b = (I + A_bb)^{-1} the diagonal blocks:
//   1. wave b forms D_b row by row, D[r][:] = e_r - A_bb[r][0:r] D[0:r][:]:
//      lane (column j, group q) keeps rows 4m + q of column j in registers,
//      each row is a partial sum per lane group and two cross-lane
//      additions;
//   2. block rows i = 1, 2, 3 in order: wave j < i forms
//      X_ij = -D_i (sum_{j <= k < i} A_ik X_kj) with fp32 16 x 16 x 4 MFMAs
//      (fp32 products, fp32 sums), the inner sum parked in a per-wave LDS
//      tile between the two products.
// Every thread of the workgroup must call it (it contains barriers); it
// starts and ends with one.  Blocks of X above the diagonal are zeroed.
#pragma once

#include "dn_mfma.h"

namespace dn {
namespace inv64 {

constexpr int SCRATCH_FLOATS = 4 * 16 * 17;  // one padded 16 x 16 tile per wave

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// A: LDS, row pitch LDA (read only).  X: LDS, row pitch LDX, disjoint from A
// and from scratch (SCRATCH_FLOATS floats).
template <int LDA, int LDX>
__device__ void inverse(const float* A, float* X, float* scratch) {
  const int t = threadIdx.x, w = t >> 6, l = t & 63, j = l & 15, q = l >> 4;
  __syncthreads();
  for (int e = t; e < 64 * 64; e += blockDim.x) {  // blocks above the diagonal
    const int r = e >> 6, c = e & 63;
    if ((c >> 4) > (r >> 4)) X[r * LDX + c] = 0.f;
  }
  if (w < 4) {  // 1. diagonal block w
    const int b0 = 16 * w;
    float d[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) d[m] = (4 * m + q == j) ? 1.f : 0.f;
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      const float* ar = A + (b0 + r) * LDA + b0;
      float p = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (4 * m + q < r) p += ar[4 * m + q] * d[m];
      p += __shfl_xor(p, 16, 64);
      p += __shfl_xor(p, 32, 64);
      if ((r & 3) == q) d[r >> 2] = (r == j ? 1.f : 0.f) - p;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) X[(b0 + 4 * m + q) * LDX + b0 + j] = d[m];
  }
  float* S = scratch + w * (16 * 17);
#pragma unroll
  for (int bi = 1; bi < 4; ++bi) {
    __syncthreads();  // block rows < bi of X are complete
    f32x4 y = zero4();
    if (w < bi) {  // Y = sum_{w <= k < bi} A_{bi,k} X_{k,w}
      for (int k = w; k < bi; ++k)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          y = mfma_f32(A[(16 * bi + j) * LDA + 16 * k + 4 * s + q],
                       X[(16 * k + 4 * s + q) * LDX + 16 * w + j], y);
#pragma unroll
      for (int e = 0; e < 4; ++e) S[(4 * q + e) * 17 + j] = y[e];
    }
    __syncthreads();  // each wave's Y tile is in its scratch
    if (w < bi) {  // X_{bi,w} = -D_bi Y
      f32x4 x = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s)
        x = mfma_f32(X[(16 * bi + j) * LDX + 16 * bi + 4 * s + q], S[(4 * s + q) * 17 + j], x);
#pragma unroll
      for (int e = 0; e < 4; ++e) X[(16 * bi + 4 * q + e) * LDX + 16 * w + j] = -x[e];
    }
  }
  __syncthreads();
}

}  // namespace inv64
}  // namespace dn
