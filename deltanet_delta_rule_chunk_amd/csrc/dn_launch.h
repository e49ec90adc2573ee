// dn_launch.h -- host-side launch descriptors between the C ABI layer and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace dn {

struct DecodeArgs {
  const void *q, *k, *v;
  const float* alpha;  // decay of the gated step, or null (plain delta rule)
  const float* beta;   // write strength, or its logit when `features` is set
  float* S;
  void* o;
  int B, H, d_k, d_v, in_dtype, out_dtype;
  hipStream_t stream;
  // Apply the layer's feature maps in-kernel: q, k are the raw projections
  // (normalise(silu(.)) is taken, the result held in in_dtype) and beta is
  // the logit (sigmoid is taken).
  bool features;
  // alpha holds d_k decays per (b, h), one per key dimension (KDA), instead
  // of one.
  bool per_dim_alpha;
};

struct FeatureArgs;

// Outputs of the chunked forward when it runs as the forward pass of the
// backward (bf16 matrix-core path, C = 128, plain form): for every 64-token
// block of the backward's workspace, X = (I + A)^{-1} of the block (the
// block's own diagonal block of the 128-token inverse), the state entering
// the block, R = V - K S from that state and Delta, row-major fp32.  o and
// S_final are then not written.
struct BwdFwdOut {
  float* ws;
  size_t block;       // floats per (head, 64-token block)
  size_t x, s, r, d;  // offsets of X [64][64], S [d_k][d_v], R [64][d_v], Delta [64][d_v]
  int nb;             // 64-token blocks per head
};

struct ChunkArgs {
  const void *q, *k, *v;
  const float* alpha;  // per-token decay of the gated form, or null (plain delta rule);
                       // [B,H,L,d_k] when per_dim_alpha
  const float* beta;
  const float* S0;  // may be null (zero state)
  void* o;
  float* S_final;   // may be null
  int B, H, L, d_k, d_v, C, in_dtype, out_dtype;
  void* workspace;  // at least chunk_workspace_bytes(...) bytes (kda_workspace_bytes)
  hipStream_t stream;
  bool per_dim_alpha;  // one decay per key dimension (KDA, dn_kda.hip)
  // bf16 matrix-core path only: apply the layer's feature maps inside the
  // WY-prep kernel, from feat's raw inputs into its outputs, which q, k and
  // beta above must then point at (the scan reads them).
  const FeatureArgs* feat = nullptr;
  // The backward's forward pass (see BwdFwdOut), or null.
  const BwdFwdOut* bwd_out = nullptr;
};

hipError_t launch_decode(const DecodeArgs& a);

// The layer's feature maps over `rows` rows of d_k (dn_features.hip).
struct FeatureArgs {
  const void *q_raw, *k_raw;
  const float* beta_logit;
  void *q_hat, *k_hat;
  float* beta;
  long long rows;
  int d_k, dtype;
  hipStream_t stream;
};
hipError_t launch_features(const FeatureArgs& a);
// Most rows one launch takes (the grid's x extent times rows per workgroup).
long long feature_max_rows(int d_k, int dtype);

// Kernel slots of the profiling hook (see deltanet_profile_start).
enum ProfSlot {
  kSlotChunkPrep = 0,
  kSlotChunkScan = 1,
  kSlotDecode = 2,
  kSlotFeatures = 3,
  kSlotBwdPrep = 4,
  kSlotBwdFwdScan = 5,
  kSlotBwdScan = 6,
  kSlotBwdCc = 7,
  kSlotBwdQk = 8,
  kNumSlots = 9
};

// Records a HIP event on `s` before (end = false) or after (end = true) the
// kernel of `slot`, when profiling is on for the calling thread; a no-op
// otherwise.
void prof_mark(int slot, bool end, hipStream_t s);

// Chunked forward: bytes of scratch it needs, and the launch sequence.
size_t chunk_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C, int in_dtype,
                             bool gated);
hipError_t launch_chunk_fwd(const ChunkArgs& a);
// Gradient of the chunked forward (dn_backward.hip).
struct BwdArgs {
  const void *q, *k, *v;    // in_dtype
  const float* beta;
  const float* S0;          // may be null (zero state)
  const float* dO;          // [B,H,L,d_v] fp32
  const float* dS_final;    // may be null (zero)
  float *dq, *dk, *dv, *dbeta;
  float* dS0;               // may be null (not written)
  int B, H, L, d_k, d_v, in_dtype;
  void* workspace;          // at least chunk_bwd_workspace_bytes(...) bytes
  hipStream_t stream;
};
size_t chunk_bwd_workspace_bytes(int B, int H, int L, int d_k, int d_v);
hipError_t launch_chunk_bwd(const BwdArgs& a);

// The per-dimension-decay (KDA) chunked forward: its workspace and launches.
size_t kda_workspace_bytes(int B, int H, int L, int d_k);
hipError_t launch_kda_chunk_fwd(const ChunkArgs& a);
// Bytes of the gated form's per-chunk log-decay table; it sits at the end of
// the workspace, after the kernels' other scratch.
size_t gated_log_decay_bytes(int B, int H, int L, int C);

// The fixed per-GPU scratch area of the allocation-free forward
// (dn_noalloc.hip): its size, and its address on the device `stream` belongs
// to (looked up on the first call for that device, then cached).
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(hipStream_t stream, void** out);

}  // namespace dn
