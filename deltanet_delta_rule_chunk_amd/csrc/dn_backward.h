// dn_backward.h -- what the backward's kernels share: the chunk size, the
// column slice of the state scans and the per-chunk workspace layout, plus
// the launches of the matrix-core state scans (dn_backward_mfma.hip) that
// replace the vector-ALU scans for bf16 q, k, v.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace dn {
namespace bwd {

constexpr int C = 64;   // chunk rows
constexpr int NT = 16;  // d_v columns per scan workgroup

// Workspace per (head, chunk), in floats; every block is row-major:
//   X = (I + A)^{-1} [C][C], M = tril(Q K^T) [C][C], dM [C][C], W [C][C],
//   S (entering state) [d_k][d_v], G' (exit gradient) [d_k][d_v],
//   R [C][d_v], Delta [C][d_v], dDelta [C][d_v].
struct Ws {
  int dk, dv;
  __host__ __device__ constexpr size_t per_chunk() const {
    return 4 * (size_t)C * C + 2 * (size_t)dk * dv + 3 * (size_t)C * dv;
  }
  __host__ __device__ constexpr size_t X() const { return 0; }
  __host__ __device__ constexpr size_t M() const { return (size_t)C * C; }
  __host__ __device__ constexpr size_t dM() const { return 2 * (size_t)C * C; }
  __host__ __device__ constexpr size_t W() const { return 3 * (size_t)C * C; }
  __host__ __device__ constexpr size_t S() const { return 4 * (size_t)C * C; }
  __host__ __device__ constexpr size_t G() const { return S() + (size_t)dk * dv; }
  __host__ __device__ constexpr size_t R() const { return G() + (size_t)dk * dv; }
  __host__ __device__ constexpr size_t D() const { return R() + (size_t)C * dv; }
  __host__ __device__ constexpr size_t dD() const { return D() + (size_t)C * dv; }
};

// M = tril(Q K^T) of every chunk on the matrix cores (bf16 q, k); X comes
// from the forward pass.  nc >= 1.
hipError_t launch_prep_mfma(int d_k, int d_v, const void* q, const void* k, int L, int nc, int bh,
                            float* ws, hipStream_t stream);

// Reverse state pass on the matrix cores (bf16 q, k): writes G'_c and
// dDelta of every chunk, dv (= dR) and dS0 (when not null).  nc >= 1.
hipError_t launch_bwd_scan_mfma(int d_k, int d_v, const void* q, const void* k,
                                const float* beta, const float* dO, const float* dS_final,
                                float* dv, float* dS0, int L, int nc, int bh, float* ws,
                                hipStream_t stream);

// The C x C gradients (dbeta) and dQ, dK in one kernel on the matrix cores
// (bf16 q, k), from the workspace the two state scans have filled.  nc >= 1.
hipError_t launch_grad_mfma(int d_k, int d_v, const void* q, const void* k, const float* beta,
                            const float* dO, const float* dv, float* dq, float* dk,
                            float* dbeta, int L, int nc, int bh, const float* ws,
                            hipStream_t stream);

}  // namespace bwd
}  // namespace dn
