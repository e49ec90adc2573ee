// dn_chunk.hip -- picks the kernel sequence for the chunked forward.
//
// bf16 inputs run on the matrix cores (dn_chunk_mfma.hip): every fp32
// operand is split into a (hi, lo) bf16 pair, which keeps the products at
// roughly fp32 accuracy.  fp32 inputs are not exact in bf16, so they run on
// the fp32 vector-ALU kernels (dn_chunk_valu.hip).
//
// Per-dimension decay (KDA) runs its own fp32 vector-ALU kernels
// (dn_kda.hip) for either input dtype.
//
// The gated form (a per-token decay alpha) runs the same kernels with the
// decay compiled in; its workspace adds, per chunk, the C within-chunk
// cumulative log-decays g_r = log(alpha_1) + ... + log(alpha_r), written by
// the prep kernel and read by the scan.

#include "dn_common.h"
#include "dn_launch.h"

namespace dn {

size_t gated_log_decay_bytes(int B, int H, int L, int C) {
  return (size_t)B * H * cdiv(L, C) * C * sizeof(float);
}

size_t chunk_workspace_bytes_valu(int B, int H, int L, int C);
hipError_t launch_chunk_fwd_valu(const ChunkArgs& a);
size_t chunk_workspace_bytes_mfma(int B, int H, int L, int C);
hipError_t launch_chunk_fwd_mfma(const ChunkArgs& a);

size_t chunk_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C, int in_dtype,
                             bool gated) {
  (void)d_k;
  (void)d_v;
  const size_t base = in_dtype == 1 ? chunk_workspace_bytes_mfma(B, H, L, C)
                                    : chunk_workspace_bytes_valu(B, H, L, C);
  return base + (gated ? gated_log_decay_bytes(B, H, L, C) : 0);
}

hipError_t launch_chunk_fwd(const ChunkArgs& a) {
  if (a.alpha && a.per_dim_alpha) return launch_kda_chunk_fwd(a);
  return a.in_dtype == 1 ? launch_chunk_fwd_mfma(a) : launch_chunk_fwd_valu(a);
}

}  // namespace dn
