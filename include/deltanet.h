/*
 * deltanet.h -- C ABI of the MI355X (gfx950) DeltaNet delta-rule library.
 *
 * The operation.  Per (batch b, head h) the state S is a d_k x d_v matrix and
 * every token t, in order, does
 *     v_old = k_t S                    (read what the state holds at key k_t)
 *     u_t   = beta_t (v_t - v_old)     (gated delta)
 *     S     = S + k_t^T u_t            (outer-product write)
 *     o_t   = q_t S                    (read after the write, no scale)
 * This is the sequential delta-rule prefill loop of the page
 * "GPT-2 から Kimi K3 まで、AI モデルの進化を解説" (news.ainew.jp), section
 * "DeltaNet (Parallelizing linear transformers with delta rule)", and, at
 * one token, that page's layer forward in "DeltaNet (Fast weight
 * programmers)".  The chunked forward computes exactly this result (up to
 * floating-point rounding) with the chunkwise-parallel generalised-Householder
 * form the same section describes.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never frees or retains them.  Tensors are dense, row-major, C-contiguous,
 *    with the shapes given below (last index fastest), 16-byte aligned.
 *  - beta and the state are always fp32.  q, k, v are fp32 or bf16
 *    (in_dtype).  o is fp32 or bf16 (out_dtype).
 *  - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *    without synchronising.  Faults during execution surface at the caller's
 *    next synchronisation.
 *  - Every argument is validated before anything is launched: on any non-OK
 *    status nothing has been launched and no output has been written.
 *  - The library keeps no state between calls besides loaded code objects;
 *    calls on different streams with disjoint buffers may run concurrently.
 */
#ifndef DELTANET_H_
#define DELTANET_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DN_OK = 0,
  DN_ERR_NULL_ARG = 1,     /* a required pointer is NULL                       */
  DN_ERR_BAD_SHAPE = 2,    /* a size is negative/zero where it must be >= 1     */
  DN_ERR_UNSUPPORTED = 3,  /* d_k, d_v, C or a dtype outside the built set      */
  DN_ERR_MISALIGNED = 4,   /* a pointer is not 16-byte aligned                  */
  DN_ERR_ALIASING = 5,     /* an output overlaps an input it must not overlap   */
  DN_ERR_WORKSPACE = 6,    /* workspace given but smaller than required         */
  DN_ERR_HIP = 7           /* a HIP runtime call failed; see deltanet_last_hip_error */
} dn_status;

/* Element types of q, k, v (in_dtype) and o (out_dtype).  The last
 * enumerator only gives the type the range of an int, so that a value
 * outside the set reaches the argument checks (DN_ERR_UNSUPPORTED). */
typedef enum { DN_F32 = 0, DN_BF16 = 1, DN_DTYPE_RANGE_ = 0x7fffffff } dn_dtype;

/*
 * Chunkwise-parallel delta-rule forward over a whole sequence.
 *
 *   q, k   : [B, H, L, d_k]   in_dtype
 *   v      : [B, H, L, d_v]   in_dtype
 *   beta   : [B, H, L]        fp32, per-token write strength
 *   S0     : [B, H, d_k, d_v] fp32 initial state, or NULL for the zero state
 *   o      : [B, H, L, d_v]   out_dtype, written (o_t read after token t's write).
 *            The kernels compute o in fp32; out_dtype = DN_BF16 stores it
 *            rounded to nearest even, which alone moves an element by up to
 *            2^-9 |o| (measured against the exact result: 1.2e-2 RMS(o) at
 *            B=4 H=12 L=2048 d=64, 2.5e-2 at B=2 H=16 L=8192 d=128 with beta
 *            = 1 heads, 1.7e-2 at B=1 H=32 L=65536 d=128, the largest errors
 *            being the roundings of the largest outputs).  Where an error
 *            bound of 2e-2 RMS(o) has to hold at such sizes, take DN_F32.
 *   S_final: [B, H, d_k, d_v] fp32 state after the last token, or NULL to skip.
 *            S_final may be the same buffer as S0 (in-place state update);
 *            any other overlap with an input is rejected.
 *   L      : any length >= 0 (L = 0 copies S0 (or zeros) to S_final; a
 *            ragged last chunk is handled by masking, an exact no-op).
 *   d_k, d_v in {64, 128}; C (chunk length) in {64, 128}.
 *   workspace: device scratch of at least deltanet_chunk_fwd_workspace_bytes()
 *            bytes, or NULL to let the library allocate and free it on
 *            `stream` (stream-ordered).  Its contents on entry do not matter.
 *
 * Returns DN_OK or the first failing check's status.
 */
int deltanet_chunk_fwd(const void* q, const void* k, const void* v, const float* beta,
                       const float* S0, void* o, float* S_final,
                       int B, int H, int L, int d_k, int d_v, int C,
                       dn_dtype in_dtype, dn_dtype out_dtype,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace deltanet_chunk_fwd needs for these sizes (0 if the
 * sizes are invalid or unsupported). */
size_t deltanet_chunk_fwd_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C,
                                          dn_dtype in_dtype);

/*
 * deltanet_chunk_fwd that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, layouts and result as
 * deltanet_chunk_fwd, without the workspace arguments: the scratch comes from
 * a fixed area of DN_NOALLOC_SCRATCH_BYTES compiled into the library, one per
 * GPU, held from the library's load until the process ends.  No call makes
 * hipMalloc, hipFree or any other allocation.
 *
 *  - Sizes whose workspace (deltanet_chunk_fwd_workspace_bytes) exceeds
 *    DN_NOALLOC_SCRATCH_BYTES return DN_ERR_WORKSPACE and launch nothing
 *    (64 MiB holds e.g. B*H = 32 heads of L = 8192 at C = 64 with bf16
 *    inputs, not the L = 65536, 32-head long-context shape).
 *  - The area is found on the device `stream` belongs to; its address is
 *    looked up (hipGetSymbolAddress) on the first call for each device, so
 *    make one call per device before capturing a graph.
 *  - All calls on one GPU share its area and it keeps the previous call's
 *    contents (nothing in it has to start cleared).  Calls that overlap in
 *    time on one GPU (other streams, other threads) race on it: serialise them.
 */
#define DN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int deltanet_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* beta,
                               const float* S0, void* o, float* S_final,
                               int B, int H, int L, int d_k, int d_v, int C,
                               dn_dtype in_dtype, dn_dtype out_dtype, hipStream_t stream);

/*
 * One decode step for B sequences x H heads (the recurrence at one token),
 * updating the state in place.
 *
 *   q, k : [B, H, d_k] in_dtype;  v : [B, H, d_v] in_dtype
 *   beta : [B, H] fp32
 *   S    : [B, H, d_k, d_v] fp32, read and overwritten with the new state
 *   o    : [B, H, d_v] out_dtype, o = q S_new
 *   d_k, d_v in {64, 128}.  o must not overlap S or any input.
 */
int deltanet_decode_step(const void* q, const void* k, const void* v, const float* beta,
                         float* S, void* o, int B, int H, int d_k, int d_v,
                         dn_dtype in_dtype, dn_dtype out_dtype, hipStream_t stream);

/*
 * Gated forms (Gated DeltaNet).  The article "How a Baseten Engineer Traced 7
 * Years of Attention Mechanism Evolution" (wpnews.pro / dev.to), section on
 * Gated DeltaNet, adds a decay alpha in [0, 1] that is applied to the old
 * state first, after which the precise delta write acts on the decayed
 * state; alpha = 1 is the plain delta rule, alpha = 0 wipes the memory.  Per
 * (b, h) and token t, in order:
 *     S     = alpha_t S
 *     v_old = k_t S
 *     u_t   = beta_t (v_t - v_old)
 *     S     = S + k_t^T u_t
 *     o_t   = q_t S
 * Arguments are those of the plain entry points plus alpha, fp32, one value
 * per token: [B, H, L] for the chunked forward, [B, H] for the decode step.
 * alpha must be 16-byte aligned and may not overlap an output; values outside
 * [0, 1] are not checked (the product is then not a decay).  A zero alpha is
 * taken as a factor of about 1e-38 inside a chunk (the kernels sum
 * log(alpha), floored at log(FLT_MIN)), which is a wipe to within fp32.
 * The chunked forward's workspace is larger than the plain one's: query it
 * with deltanet_gated_chunk_fwd_workspace_bytes().  With L = 0, alpha may be
 * NULL.  Status codes and every other rule are as for the plain calls.
 */
int deltanet_gated_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const float* S0, void* o, float* S_final,
                             int B, int H, int L, int d_k, int d_v, int C,
                             dn_dtype in_dtype, dn_dtype out_dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace deltanet_gated_chunk_fwd needs (0 if the sizes are
 * invalid or unsupported). */
size_t deltanet_gated_chunk_fwd_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C,
                                                dn_dtype in_dtype);

/* One gated decode step, S updated in place; o = q S_new.  alpha: [B, H] fp32. */
int deltanet_gated_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, float* S, void* o, int B, int H,
                               int d_k, int d_v, dn_dtype in_dtype, dn_dtype out_dtype,
                               hipStream_t stream);

/*
 * Gradient of the chunked forward (training).  The pages present the chunked
 * form as the way to train the delta rule in linear time but print no
 * backward pass; this one is the reverse-mode derivative of the forward
 * above (plain delta rule, no gate).  Given the gradients of a loss with
 * respect to the forward's outputs, it returns those with respect to its
 * inputs:
 *   q, k   : [B, H, L, d_k]  in_dtype;   v : [B, H, L, d_v] in_dtype
 *   beta   : [B, H, L] fp32;  S0 : [B, H, d_k, d_v] fp32 or NULL (zero state)
 *   dO     : [B, H, L, d_v] fp32, dL/do
 *   dS_final: [B, H, d_k, d_v] fp32, dL/dS_final, or NULL (zero)
 *   dq, dk : [B, H, L, d_k] fp32;  dv : [B, H, L, d_v] fp32;
 *   dbeta  : [B, H, L] fp32;       dS0 : [B, H, d_k, d_v] fp32 or NULL (not
 *            written)
 * The forward is recomputed inside (nothing from a previous forward call is
 * needed).  64-token chunks whatever C names (C must still be 64 or 128);
 * with bf16 inputs the recomputed forward runs on the chunked forward's
 * kernels at 128-token chunks.  bf16 inputs run every product on bf16 matrix
 * cores with each fp32 operand split into a (hi, lo) bf16 pair; fp32 inputs
 * run fp32 vector-ALU kernels.  Outputs may not overlap inputs or one
 * another.  The workspace holds, per 64-token chunk, the entering state and
 * the exit gradient (2 d_k d_v floats) besides per-chunk matrices, and the
 * forward's T per 128-token chunk: query deltanet_chunk_bwd_workspace_bytes().
 */
int deltanet_chunk_bwd(const void* q, const void* k, const void* v, const float* beta,
                       const float* S0, const float* dO, const float* dS_final,
                       float* dq, float* dk, float* dv, float* dbeta, float* dS0,
                       int B, int H, int L, int d_k, int d_v, int C, dn_dtype in_dtype,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace deltanet_chunk_bwd needs (0 if the sizes are invalid or
 * unsupported). */
size_t deltanet_chunk_bwd_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C,
                                          dn_dtype in_dtype);

/*
 * Per-dimension decay (KDA).  The same article describes Kimi Linear's KDA as
 * Gated DeltaNet with the scalar gate turned into a vector: each dimension of
 * the memory forgets at its own rate.  The gate acts on the key dimension,
 * the rows of S.  Per (b, h) and token t, in order:
 *     S     = diag(alpha_t) S          alpha_t in [0, 1]^{d_k}
 *     v_old = k_t S
 *     u_t   = beta_t (v_t - v_old)
 *     S     = S + k_t^T u_t
 *     o_t   = q_t S
 * Arguments are those of the gated entry points with alpha one fp32 per key
 * dimension: [B, H, L, d_k] for the chunked forward, [B, H, d_k] for the
 * decode step.  alpha must be 16-byte aligned and may not overlap an output;
 * zeros are floored inside a chunk as for the scalar gate.  The chunked
 * forward runs in 64-token chunks whatever C names (the result does not
 * depend on the chunk size; C must still be 64 or 128): for bf16 inputs its
 * scan and most of its prep on bf16 matrix cores with split operands, for
 * fp32 inputs on fp32 vector-ALU kernels.  Its workspace is larger than the other forms':
 * query deltanet_kda_chunk_fwd_workspace_bytes().  With L = 0, alpha may be
 * NULL.
 */
int deltanet_kda_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* S0, void* o, float* S_final,
                           int B, int H, int L, int d_k, int d_v, int C,
                           dn_dtype in_dtype, dn_dtype out_dtype,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace deltanet_kda_chunk_fwd needs (0 if the sizes are invalid
 * or unsupported). */
size_t deltanet_kda_chunk_fwd_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C,
                                              dn_dtype in_dtype);

/* One decode step with per-dimension decay, S updated in place; o = q S_new.
 * alpha: [B, H, d_k] fp32. */
int deltanet_kda_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, float* S, void* o, int B, int H,
                             int d_k, int d_v, dn_dtype in_dtype, dn_dtype out_dtype,
                             hipStream_t stream);

/*
 * The layer's feature maps (page "GPT-2 から Kimi K3 まで、AI モデルの進化を解説",
 * section "DeltaNet (Fast weight programmers)": before the delta rule the
 * layer maps its projections to
 *     q = normalise(silu(q_raw)),  k = normalise(silu(k_raw)),
 *     beta = sigmoid(beta_logit),
 * with silu(x) = x sigmoid(x) and normalise(x) = x / max(||x||_2, 1e-12)
 * along d_k, as PyTorch's F.normalize).  The maps are evaluated in fp32; q
 * and k are stored in `dtype` (bf16: rounded to nearest, ties to even),
 * beta in fp32.  Elements of a row beyond ~1e19 overflow its fp32 sum of
 * squares (the row then maps to zeros).
 *
 *   q_raw, k_raw, q_hat, k_hat : [B, H, L, d_k] dtype
 *   beta_logit, beta            : [B, H, L] fp32
 *   d_k in {64, 128}.  Every pointer is required when B H L > 0.  An output
 *   may be the very buffer of its own input (in place); any other overlap is
 *   rejected.
 */
int deltanet_feature_prep(const void* q_raw, const void* k_raw, const float* beta_logit,
                          void* q_hat, void* k_hat, float* beta,
                          int B, int H, int L, int d_k, dn_dtype dtype, hipStream_t stream);

/*
 * The chunked forward fed by the raw projections: the feature maps above,
 * then the plain (alpha == NULL) or gated (alpha given) chunked forward on the
 * mapped q, k, beta.  Arguments are those of deltanet_chunk_fwd /
 * deltanet_gated_chunk_fwd with q_raw, k_raw in place of q, k and
 * beta_logit in place of beta.  The mapped operands live in the workspace,
 * which is therefore larger: query it with
 * deltanet_chunk_fwd_features_workspace_bytes(..., gated = alpha != NULL).
 */
int deltanet_chunk_fwd_features(const void* q_raw, const void* k_raw, const void* v,
                                const float* alpha, const float* beta_logit, const float* S0,
                                void* o, float* S_final,
                                int B, int H, int L, int d_k, int d_v, int C,
                                dn_dtype in_dtype, dn_dtype out_dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace deltanet_chunk_fwd_features needs (gated != 0 when
 * alpha will be given; 0 if the sizes are invalid or unsupported). */
size_t deltanet_chunk_fwd_features_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C,
                                                   dn_dtype in_dtype, int gated);

/*
 * One decode step fed by the raw projections: the feature maps are applied
 * inside the step's kernel (no extra memory traffic), then the plain
 * (alpha == NULL) or gated step.  Arguments are those of
 * deltanet_decode_step / deltanet_gated_decode_step with q_raw, k_raw and
 * beta_logit in place of q, k and beta.
 */
int deltanet_decode_step_features(const void* q_raw, const void* k_raw, const void* v,
                                  const float* alpha, const float* beta_logit, float* S, void* o,
                                  int B, int H, int d_k, int d_v, dn_dtype in_dtype, dn_dtype out_dtype,
                                  hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* deltanet_status_string(int status);

/* The hipError_t behind the last DN_ERR_HIP returned on this thread (0 if none). */
int deltanet_last_hip_error(void);

/*
 * Profiling hook.  Between deltanet_profile_start() and
 * deltanet_profile_stop() on the same host thread, every kernel the library
 * launches from that thread is bracketed by two HIP events recorded on the
 * call's stream.  deltanet_profile_stop() waits for those events and writes,
 * per kernel slot, the summed elapsed milliseconds and the launch count
 * (nslots entries each; slots: 0 = chunk WY-prep kernel, 1 = chunk scan
 * kernel, 2 = decode kernel, 3 = feature-map kernel; the backward's kernels:
 * 4 = prep, 5 = forward state pass (for bf16 inputs the chunked forward's
 * prep and scan kernels at 128-token chunks, counted together), 6 = reverse
 * state pass, 7 = per-chunk matrix gradients, 8 = dq / dk; for bf16 inputs one
 * kernel computes both the matrix gradients and dq / dk and is counted in
 * slot 8).  Recording adds two
 * event records per launch.
 * deltanet_profile_start() creates the thread's events up front (4096,
 * enough for 2048 launches; more are created as needed), so it can take a
 * few milliseconds the first time; it returns DN_ERR_HIP if that fails.
 */
int deltanet_profile_start(void);
int deltanet_profile_stop(double* ms_per_slot, int* launches_per_slot, int nslots);

/* Library version as major*10000 + minor*100 + patch. */
int deltanet_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DELTANET_H_ */
