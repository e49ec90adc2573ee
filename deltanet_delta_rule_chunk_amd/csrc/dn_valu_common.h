// dn_valu_common.h -- pieces shared by the fp32 vector-ALU chunk kernels
// (dn_chunk_valu.hip, dn_kda.hip): staging rows into LDS and the blocked
// inverse of a unit lower-triangular matrix.  Every function is called by all
// threads of a workgroup.
#pragma once

#include "dn_common.h"

namespace dn {
namespace valu {

constexpr int BS = 16;  // block size of the blocked triangular inverse

// rows x cols of a row-major source (row pitch cols) into LDS (row pitch
// ld), as fp32; rows at or past rows_valid read as zero.
template <typename IT>
__device__ __forceinline__ void load_rows(float* dst, int ld, const IT* src, int rows_valid,
                                          int rows, int cols) {
  for (int e = threadIdx.x; e < rows * cols; e += blockDim.x) {
    const int r = e / cols, c = e % cols;
    dst[r * ld + c] = r < rows_valid ? to_f32(src[(size_t)r * cols + c]) : 0.f;
  }
}

// X = (I + A)^{-1} for a strictly lower-triangular C x C matrix A (LDS, row
// pitch lda, read only), into X (LDS, row pitch ldx), by 16 x 16 blocks:
//   diagonal blocks by forward substitution (column j of a block depends
//   only on the block's earlier rows of column j);
//   off-diagonal block rows in order, X_ij = -X_ii sum_{j <= k < i} A_ik X_kj.
// Expects blockDim.x >= BS * BS (each thread then holds at most C / BS - 1
// pending outputs of a block row).  Starts and ends with a barrier.
template <int C>
__device__ void unit_lower_inverse(const float* A, int lda, float* X, int ldx) {
  constexpr int NB = C / BS;
  __syncthreads();
  for (int e = threadIdx.x; e < C * C; e += blockDim.x) X[(e / C) * ldx + e % C] = 0.f;
  __syncthreads();
  for (int t = threadIdx.x; t < C; t += blockDim.x) {
    const int j = t, blk_end = (j / BS + 1) * BS;
    X[j * ldx + j] = 1.f;
    for (int r = j + 1; r < blk_end; ++r) {
      float acc = 0.f;
      for (int i = j; i < r; ++i) acc += A[r * lda + i] * X[i * ldx + j];
      X[r * ldx + j] = -acc;
    }
  }
  __syncthreads();
  for (int bi = 1; bi < NB; ++bi) {
    // Y_j = sum_k A_ik X_kj, parked in X_ij's slot.
    for (int e = threadIdx.x; e < bi * BS * BS; e += blockDim.x) {
      const int bj = e / (BS * BS), rr = (e / BS) % BS, cc = e % BS;
      const int row = bi * BS + rr, col = bj * BS + cc;
      float acc = 0.f;
      for (int m = bj * BS; m < bi * BS; ++m) acc += A[row * lda + m] * X[m * ldx + col];
      X[row * ldx + col] = acc;
    }
    __syncthreads();
    float out[NB];
    for (int e = threadIdx.x, s = 0; e < bi * BS * BS; e += blockDim.x, ++s) {
      const int bj = e / (BS * BS), rr = (e / BS) % BS, cc = e % BS;
      const int row = bi * BS + rr, col = bj * BS + cc;
      float acc = 0.f;
      for (int m = 0; m < BS; ++m) acc += X[row * ldx + bi * BS + m] * X[(bi * BS + m) * ldx + col];
      out[s] = -acc;
    }
    __syncthreads();
    for (int e = threadIdx.x, s = 0; e < bi * BS * BS; e += blockDim.x, ++s) {
      const int bj = e / (BS * BS), rr = (e / BS) % BS, cc = e % BS;
      X[(bi * BS + rr) * ldx + bj * BS + cc] = out[s];
    }
    __syncthreads();
  }
}

}  // namespace valu
}  // namespace dn
