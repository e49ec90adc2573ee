// dn_chunk.hip -- chooses the kernel sequence for the chunked forward.

#include "dn_common.h"
#include "dn_launch.h"

namespace dn {

size_t chunk_workspace_bytes_valu(int B, int H, int L, int C);
hipError_t launch_chunk_fwd_valu(const ChunkArgs& a);

size_t chunk_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C, int in_dtype) {
  (void)d_k; (void)d_v; (void)in_dtype;
  return chunk_workspace_bytes_valu(B, H, L, C);
}

hipError_t launch_chunk_fwd(const ChunkArgs& a) { return launch_chunk_fwd_valu(a); }

}  // namespace dn
