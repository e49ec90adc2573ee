// dn_kda.h -- what the per-dimension-decay (KDA) kernels share: the chunk
// size, the column slice of the scan and the per-chunk workspace layout, and
// the launches of the matrix-core prep and scan (dn_kda_mfma.hip) that
// replace the vector-ALU kernels for bf16 q, k, v.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace dn {
namespace kda {

constexpr int C = 64;   // chunk rows
constexpr int NT = 16;  // d_v columns per scan workgroup

// Workspace per (head, chunk), in floats, each block row-major: T, P
// (C x C each), K o e^g, Q o e^g, K o e^{g_C - g} (C x d_k each), e^{g_C}
// (d_k).  The vector-ALU prep stores the matrix blocks in fp32; the
// matrix-core prep stores each as its split pair, a bf16 plane of hi =
// bf16(x) followed by one of lo = bf16(x - hi), in the same bytes.
__host__ __device__ constexpr size_t chunk_floats(int dk) {
  return 2 * (size_t)C * C + 3 * (size_t)C * dk + dk;
}

// The prep on the matrix cores for bf16 q, k (the tiles of A and P below
// the 16-row block diagonal): fills the workspace of every chunk.  nc >= 1.
hipError_t launch_prep_mfma(int d_k, const void* q, const void* k, const float* alpha,
                            const float* beta, int L, int nc, int bh, float* ws,
                            hipStream_t stream);

// The scan over chunks on the matrix cores, from the workspace the prep
// kernel has filled: o (out_dtype 0 = fp32, 1 = bf16) and S_final (when not
// null).  v is bf16.  nc = ceil(L / C) >= 0; bh = B * H.
hipError_t launch_scan_mfma(int d_k, int d_v, int out_dtype, const void* v, const float* S0,
                            void* o, float* S_final, int L, int nc, int bh, const float* ws,
                            hipStream_t stream);

}  // namespace kda
}  // namespace dn
