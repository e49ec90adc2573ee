// dn_api.cpp -- the C ABI of libdeltanet (declared in include/deltanet.h).
//
// Every entry point validates all of its arguments on the host before it
// touches the HIP runtime: a failing check returns a status, launches nothing
// and writes nothing.  This also means the validation paths run (and are
// tested) on machines with no GPU.

#include "deltanet.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "dn_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kVersion = 500;  // 0.5.0

int hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return DN_ERR_HIP;
}

bool dtype_ok(int t) { return t == DN_F32 || t == DN_BF16; }
size_t dtype_size(int t) { return t == DN_F32 ? 4 : 2; }
bool dim_ok(int d) { return d == 64 || d == 128; }
bool chunk_ok(int c) { return c == 64 || c == 128; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  const void* p;
  size_t n;  // bytes
};

bool overlap(Span a, Span b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

struct ChunkSizes {
  size_t qk, v, beta, o, state;
};

// Returns DN_OK and fills sizes, or the status of the first failed check.
int check_chunk_shape(int B, int H, int L, int d_k, int d_v, int C, int in_dtype,
                      int out_dtype, ChunkSizes* s) {
  if (B < 1 || H < 1 || L < 0 || d_k < 1 || d_v < 1 || C < 1) return DN_ERR_BAD_SHAPE;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return DN_ERR_UNSUPPORTED;
  if (!dim_ok(d_k) || !dim_ok(d_v) || !chunk_ok(C)) return DN_ERR_UNSUPPORTED;
  // Grid limits: heads go in grid y (<= 65535); chunk count in grid x.
  if ((int64_t)B * H > 65535) return DN_ERR_UNSUPPORTED;
  const size_t tok = (size_t)B * H * (size_t)L;
  s->qk = tok * d_k * dtype_size(in_dtype);
  s->v = tok * d_v * dtype_size(in_dtype);
  s->beta = tok * sizeof(float);
  s->o = tok * d_v * dtype_size(out_dtype);
  s->state = (size_t)B * H * d_k * d_v * sizeof(float);
  return DN_OK;
}

// Profiling hook state (per thread): pairs of events around each kernel.
struct ProfRecord {
  int slot;
  hipEvent_t begin, end;
};
struct ProfState {
  bool on = false;
  std::vector<ProfRecord> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t pending = nullptr;
  int pending_slot = -1;
  hipError_t error = hipSuccess;
};
thread_local ProfState g_prof;
// Events kept ready by deltanet_profile_start (two per bracketed launch).
constexpr size_t kProfPoolEvents = 4096;

hipEvent_t prof_event() {
  if (!g_prof.pool.empty()) {
    hipEvent_t e = g_prof.pool.back();
    g_prof.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  hipError_t r = hipEventCreate(&e);
  if (r != hipSuccess && g_prof.error == hipSuccess) g_prof.error = r;
  return r == hipSuccess ? e : nullptr;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace of the chunked forward: the chunk kernels' scratch, then (with
// the feature maps) the mapped q, k and beta, each 256-byte aligned.
struct WsLayout {
  size_t core, qk, beta, total;
};
WsLayout ws_layout(int B, int H, int L, int d_k, int d_v, int C, int in_dtype, bool gated,
                   bool features, const ChunkSizes& s) {
  WsLayout w{dn::chunk_workspace_bytes(B, H, L, d_k, d_v, C, in_dtype, gated), 0, 0, 0};
  if (features) {
    w.core = align256(w.core);
    w.qk = align256(s.qk);
    w.beta = align256(s.beta);
  }
  w.total = w.core + 2 * w.qk + w.beta;
  return w;
}

// Shared body of the chunked forwards: plain (alpha = null) or gated, on
// mapped operands or (features) on the raw projections, in which case q, k
// are the raw q, k and beta holds the logits.
int chunk_fwd_impl(const void* q, const void* k, const void* v, const float* alpha,
                   const float* beta, const float* S0, void* o, float* S_final, int B, int H,
                   int L, int d_k, int d_v, int C, int in_dtype, int out_dtype, void* workspace,
                   size_t workspace_bytes, hipStream_t stream, bool features = false,
                   bool per_dim = false, bool fixed_scratch = false) {
  ChunkSizes s;
  int st = check_chunk_shape(B, H, L, d_k, d_v, C, in_dtype, out_dtype, &s);
  if (st != DN_OK) return st;
  if (L > 0 && (!q || !k || !v || !beta || !o)) return DN_ERR_NULL_ARG;
  if (features && (long long)B * H * L > dn::feature_max_rows(d_k, in_dtype))
    return DN_ERR_UNSUPPORTED;
  const bool gated = alpha != nullptr;
  const void* ptrs[] = {q, k, v, alpha, beta, S0, o, S_final, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return DN_ERR_MISALIGNED;

  const size_t alpha_bytes = per_dim ? s.beta * d_k : s.beta;
  const Span sq{q, s.qk}, sk{k, s.qk}, sv{v, s.v}, sa{alpha, alpha_bytes}, sb{beta, s.beta};
  const Span ss0{S0, s.state}, so{o, s.o}, ssf{S_final, s.state};
  const WsLayout wl = ws_layout(B, H, L, d_k, d_v, C, in_dtype, gated, features, s);
  const size_t need = per_dim ? dn::kda_workspace_bytes(B, H, L, d_k) : wl.total;
  const Span sw{workspace, workspace ? need : 0};
  for (Span in : {sq, sk, sv, sa, sb, ss0})
    if (overlap(so, in) || (in.p != S0 && overlap(ssf, in))) return DN_ERR_ALIASING;
  if (overlap(so, ssf)) return DN_ERR_ALIASING;
  if (S_final && S0 && S_final != S0 && overlap(ssf, ss0)) return DN_ERR_ALIASING;
  for (Span x : {sq, sk, sv, sa, sb, ss0, so, ssf})
    if (overlap(sw, x)) return DN_ERR_ALIASING;
  if (workspace && workspace_bytes < need) return DN_ERR_WORKSPACE;
  if (fixed_scratch && need > dn::kNoallocScratchBytes) return DN_ERR_WORKSPACE;

  void* ws = workspace;
  if (fixed_scratch && need > 0) {
    hipError_t e = dn::noalloc_scratch(stream, &ws);
    if (e != hipSuccess) return hip_fail(e);
  }
  const bool own_ws = (ws == nullptr && need > 0);
  if (own_ws) {
    hipError_t e = hipMallocAsync(&ws, need, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  hipError_t e = hipSuccess;
  dn::FeatureArgs f{};
  // The bf16 matrix-core path maps q, k and beta inside its WY-prep kernel;
  // the other paths run the streaming feature kernel first.
  const bool fused_maps = features && L > 0 && in_dtype == DN_BF16 && !per_dim;
  if (features && L > 0) {
    char* base = static_cast<char*>(ws) + wl.core;
    void *qh = base, *kh = base + wl.qk;
    float* bh = reinterpret_cast<float*>(base + 2 * wl.qk);
    f = dn::FeatureArgs{q, k, beta, qh, kh, bh, (long long)B * H * L, d_k, in_dtype, stream};
    if (!fused_maps) e = dn::launch_features(f);
    q = qh;
    k = kh;
    beta = bh;
  }
  if (e == hipSuccess) {
    dn::ChunkArgs a{q, k, v, alpha, beta, S0, o, S_final, B, H, L, d_k, d_v, C, in_dtype,
                    out_dtype, ws, stream, per_dim};
    if (fused_maps) a.feat = &f;
    e = dn::launch_chunk_fwd(a);
  }
  if (own_ws) {
    hipError_t f = hipFreeAsync(ws, stream);
    if (e == hipSuccess) e = f;
  }
  if (e != hipSuccess) return hip_fail(e);
  return DN_OK;
}

// Shared body of the plain (alpha = null) and gated decode steps.
int decode_impl(const void* q, const void* k, const void* v, const float* alpha,
                const float* beta, float* S, void* o, int B, int H, int d_k, int d_v,
                int in_dtype, int out_dtype, hipStream_t stream, bool features = false,
                bool per_dim = false) {
  if (B < 1 || H < 1 || d_k < 1 || d_v < 1) return DN_ERR_BAD_SHAPE;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return DN_ERR_UNSUPPORTED;
  if (!dim_ok(d_k) || !dim_ok(d_v)) return DN_ERR_UNSUPPORTED;
  if ((int64_t)B * H > 0x7fffffff) return DN_ERR_UNSUPPORTED;
  if (!q || !k || !v || !beta || !S || !o) return DN_ERR_NULL_ARG;
  const void* ptrs[] = {q, k, v, alpha, beta, S, o};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return DN_ERR_MISALIGNED;
  const size_t bh = (size_t)B * H;
  const Span sq{q, bh * d_k * dtype_size(in_dtype)}, sk{k, sq.n};
  const Span sv{v, bh * d_v * dtype_size(in_dtype)}, sb{beta, bh * sizeof(float)};
  const Span sa{alpha, bh * sizeof(float) * (per_dim ? d_k : 1)};
  const Span sS{S, bh * d_k * d_v * sizeof(float)}, so{o, bh * d_v * dtype_size(out_dtype)};
  for (Span in : {sq, sk, sv, sa, sb, sS})
    if (overlap(so, in)) return DN_ERR_ALIASING;
  for (Span in : {sq, sk, sv, sa, sb})
    if (overlap(sS, in)) return DN_ERR_ALIASING;

  dn::DecodeArgs a{q, k, v, alpha, beta, S, o, B, H, d_k, d_v, in_dtype, out_dtype, stream,
                   features, per_dim};
  hipError_t e = dn::launch_decode(a);
  if (e != hipSuccess) return hip_fail(e);
  return DN_OK;
}

}  // namespace

namespace dn {

void prof_mark(int slot, bool end, hipStream_t s) {
  if (!g_prof.on) return;
  hipEvent_t e = prof_event();
  if (!e) return;
  hipError_t r = hipEventRecord(e, s);
  if (r != hipSuccess && g_prof.error == hipSuccess) g_prof.error = r;
  if (!end) {
    g_prof.pending = e;
    g_prof.pending_slot = slot;
  } else if (g_prof.pending && g_prof.pending_slot == slot) {
    g_prof.recs.push_back({slot, g_prof.pending, e});
    g_prof.pending = nullptr;
  } else {
    g_prof.pool.push_back(e);
  }
}

}  // namespace dn

extern "C" {

int deltanet_profile_start(void) {
  for (const ProfRecord& r : g_prof.recs) {
    g_prof.pool.push_back(r.begin);
    g_prof.pool.push_back(r.end);
  }
  g_prof.recs.clear();
  g_prof.pending = nullptr;
  g_prof.error = hipSuccess;
  // Create the events up front: creating one between a kernel's launch and
  // its closing record can leave the GPU waiting on the host, and that wait
  // would be counted as the kernel's time.
  while (g_prof.pool.size() < kProfPoolEvents) {
    hipEvent_t e = nullptr;
    const hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) return hip_fail(r);
    g_prof.pool.push_back(e);
  }
  g_prof.on = true;
  return DN_OK;
}

int deltanet_profile_stop(double* ms_per_slot, int* launches_per_slot, int nslots) {
  g_prof.on = false;
  if (nslots < 0 || (nslots > 0 && (!ms_per_slot || !launches_per_slot))) return DN_ERR_NULL_ARG;
  for (int i = 0; i < nslots; ++i) {
    ms_per_slot[i] = 0.0;
    launches_per_slot[i] = 0;
  }
  if (g_prof.error != hipSuccess) return hip_fail(g_prof.error);
  for (const ProfRecord& r : g_prof.recs) {
    hipError_t e = hipEventSynchronize(r.end);
    if (e != hipSuccess) return hip_fail(e);
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.begin, r.end);
    if (e != hipSuccess) return hip_fail(e);
    if (r.slot >= 0 && r.slot < nslots) {
      ms_per_slot[r.slot] += ms;
      launches_per_slot[r.slot] += 1;
    }
  }
  return DN_OK;
}

int deltanet_version(void) { return kVersion; }

int deltanet_last_hip_error(void) { return g_last_hip_error; }

const char* deltanet_status_string(int status) {
  switch (status) {
    case DN_OK: return "ok";
    case DN_ERR_NULL_ARG: return "a required pointer is NULL";
    case DN_ERR_BAD_SHAPE: return "invalid size (B, H, d_k, d_v, C must be >= 1; L >= 0)";
    case DN_ERR_UNSUPPORTED:
      return "unsupported configuration (d_k, d_v in {64,128}; C in {64,128}; dtype f32/bf16; B*H <= 65535)";
    case DN_ERR_MISALIGNED: return "a tensor pointer is not 16-byte aligned";
    case DN_ERR_ALIASING: return "an output overlaps an input";
    case DN_ERR_WORKSPACE: return "workspace smaller than the matching *_workspace_bytes() query";
    case DN_ERR_HIP: return "HIP runtime error (see deltanet_last_hip_error)";
    default: return "unknown status";
  }
}

int deltanet_feature_prep(const void* q_raw, const void* k_raw, const float* beta_logit,
                          void* q_hat, void* k_hat, float* beta, int B, int H, int L, int d_k,
                          dn_dtype dtype, hipStream_t stream) {
  if (B < 1 || H < 1 || L < 0 || d_k < 1) return DN_ERR_BAD_SHAPE;
  if (!dtype_ok(dtype) || !dim_ok(d_k)) return DN_ERR_UNSUPPORTED;
  const long long rows = (long long)B * H * L;
  if (rows > dn::feature_max_rows(d_k, dtype)) return DN_ERR_UNSUPPORTED;
  if (rows == 0) return DN_OK;
  if (!q_raw || !k_raw || !beta_logit || !q_hat || !k_hat || !beta) return DN_ERR_NULL_ARG;
  const void* ptrs[] = {q_raw, k_raw, beta_logit, q_hat, k_hat, beta};
  for (const void* p : ptrs)
    if (!aligned16(p)) return DN_ERR_MISALIGNED;
  const size_t nqk = (size_t)rows * d_k * dtype_size(dtype), nb = (size_t)rows * sizeof(float);
  const Span in[] = {{q_raw, nqk}, {k_raw, nqk}, {beta_logit, nb}};
  const Span out[] = {{q_hat, nqk}, {k_hat, nqk}, {beta, nb}};
  // An output may be its own input (the maps run in place) and must
  // overlap nothing else.
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlap(out[i], in[j]) && !(i == j && out[i].p == in[j].p)) return DN_ERR_ALIASING;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(out[i], out[j])) return DN_ERR_ALIASING;
  }
  dn::FeatureArgs f{q_raw, k_raw, beta_logit, q_hat, k_hat, beta, rows, d_k, dtype, stream};
  hipError_t e = dn::launch_features(f);
  if (e != hipSuccess) return hip_fail(e);
  return DN_OK;
}

size_t deltanet_chunk_fwd_features_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C,
                                                   dn_dtype in_dtype, int gated) {
  ChunkSizes s;
  if (check_chunk_shape(B, H, L, d_k, d_v, C, in_dtype, DN_F32, &s) != DN_OK) return 0;
  return ws_layout(B, H, L, d_k, d_v, C, in_dtype, gated != 0, true, s).total;
}

int deltanet_chunk_fwd_features(const void* q_raw, const void* k_raw, const void* v,
                                const float* alpha, const float* beta_logit, const float* S0,
                                void* o, float* S_final, int B, int H, int L, int d_k, int d_v,
                                int C, dn_dtype in_dtype, dn_dtype out_dtype, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return chunk_fwd_impl(q_raw, k_raw, v, alpha, beta_logit, S0, o, S_final, B, H, L, d_k, d_v, C,
                        in_dtype, out_dtype, workspace, workspace_bytes, stream, true);
}

int deltanet_decode_step_features(const void* q_raw, const void* k_raw, const void* v,
                                  const float* alpha, const float* beta_logit, float* S, void* o,
                                  int B, int H, int d_k, int d_v, dn_dtype in_dtype, dn_dtype out_dtype,
                                  hipStream_t stream) {
  return decode_impl(q_raw, k_raw, v, alpha, beta_logit, S, o, B, H, d_k, d_v, in_dtype,
                     out_dtype, stream, true);
}

size_t deltanet_chunk_bwd_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C,
                                          dn_dtype in_dtype) {
  ChunkSizes s;
  if (check_chunk_shape(B, H, L, d_k, d_v, C, in_dtype, DN_F32, &s) != DN_OK) return 0;
  return dn::chunk_bwd_workspace_bytes(B, H, L, d_k, d_v);
}

int deltanet_chunk_bwd(const void* q, const void* k, const void* v, const float* beta,
                       const float* S0, const float* dO, const float* dS_final, float* dq,
                       float* dk, float* dv, float* dbeta, float* dS0, int B, int H, int L,
                       int d_k, int d_v, int C, dn_dtype in_dtype, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  ChunkSizes s;
  int st = check_chunk_shape(B, H, L, d_k, d_v, C, in_dtype, DN_F32, &s);
  if (st != DN_OK) return st;
  if (L > 0 && (!q || !k || !v || !beta || !dO || !dq || !dk || !dv || !dbeta))
    return DN_ERR_NULL_ARG;
  const void* ptrs[] = {q, k, v, beta, S0, dO, dS_final, dq, dk, dv, dbeta, dS0, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return DN_ERR_MISALIGNED;
  const size_t tok = (size_t)B * H * (size_t)L;
  const Span in[] = {{q, s.qk}, {k, s.qk}, {v, s.v}, {beta, s.beta}, {S0, s.state},
                     {dO, tok * d_v * 4}, {dS_final, s.state}};
  const Span out[] = {{dq, tok * d_k * 4}, {dk, tok * d_k * 4}, {dv, tok * d_v * 4},
                      {dbeta, s.beta}, {dS0, s.state}};
  const size_t need = dn::chunk_bwd_workspace_bytes(B, H, L, d_k, d_v);
  const Span sw{workspace, workspace ? need : 0};
  for (int i = 0; i < 5; ++i) {
    for (const Span& x : in)
      if (overlap(out[i], x)) return DN_ERR_ALIASING;
    for (int j = i + 1; j < 5; ++j)
      if (overlap(out[i], out[j])) return DN_ERR_ALIASING;
    if (overlap(sw, out[i])) return DN_ERR_ALIASING;
  }
  for (const Span& x : in)
    if (overlap(sw, x)) return DN_ERR_ALIASING;
  if (workspace && workspace_bytes < need) return DN_ERR_WORKSPACE;

  void* ws = workspace;
  const bool own_ws = (ws == nullptr && need > 0);
  if (own_ws) {
    hipError_t e = hipMallocAsync(&ws, need, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  dn::BwdArgs a{q,  k,  v,     beta, S0, dO, dS_final, dq,        dk, dv, dbeta,
                dS0, B, H, L, d_k, d_v, in_dtype, ws, stream};
  hipError_t e = dn::launch_chunk_bwd(a);
  if (own_ws) {
    hipError_t f = hipFreeAsync(ws, stream);
    if (e == hipSuccess) e = f;
  }
  if (e != hipSuccess) return hip_fail(e);
  return DN_OK;
}

size_t deltanet_kda_chunk_fwd_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C,
                                              dn_dtype in_dtype) {
  ChunkSizes s;
  if (check_chunk_shape(B, H, L, d_k, d_v, C, in_dtype, DN_F32, &s) != DN_OK) return 0;
  return dn::kda_workspace_bytes(B, H, L, d_k);
}

int deltanet_kda_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* S0, void* o, float* S_final, int B,
                           int H, int L, int d_k, int d_v, int C, dn_dtype in_dtype, dn_dtype out_dtype,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (L > 0 && !alpha) return DN_ERR_NULL_ARG;
  return chunk_fwd_impl(q, k, v, alpha, beta, S0, o, S_final, B, H, L, d_k, d_v, C, in_dtype,
                        out_dtype, workspace, workspace_bytes, stream, false, true);
}

int deltanet_kda_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, float* S, void* o, int B, int H, int d_k,
                             int d_v, dn_dtype in_dtype, dn_dtype out_dtype, hipStream_t stream) {
  if (!alpha) return DN_ERR_NULL_ARG;
  return decode_impl(q, k, v, alpha, beta, S, o, B, H, d_k, d_v, in_dtype, out_dtype, stream,
                     false, true);
}

size_t deltanet_chunk_fwd_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C,
                                          dn_dtype in_dtype) {
  ChunkSizes s;
  if (check_chunk_shape(B, H, L, d_k, d_v, C, in_dtype, DN_F32, &s) != DN_OK) return 0;
  return dn::chunk_workspace_bytes(B, H, L, d_k, d_v, C, in_dtype, false);
}

size_t deltanet_gated_chunk_fwd_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C,
                                                dn_dtype in_dtype) {
  ChunkSizes s;
  if (check_chunk_shape(B, H, L, d_k, d_v, C, in_dtype, DN_F32, &s) != DN_OK) return 0;
  return dn::chunk_workspace_bytes(B, H, L, d_k, d_v, C, in_dtype, true);
}

int deltanet_chunk_fwd(const void* q, const void* k, const void* v, const float* beta,
                       const float* S0, void* o, float* S_final, int B, int H, int L, int d_k,
                       int d_v, int C, dn_dtype in_dtype, dn_dtype out_dtype, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  return chunk_fwd_impl(q, k, v, nullptr, beta, S0, o, S_final, B, H, L, d_k, d_v, C, in_dtype,
                        out_dtype, workspace, workspace_bytes, stream);
}

int deltanet_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* beta,
                               const float* S0, void* o, float* S_final, int B, int H, int L,
                               int d_k, int d_v, int C, dn_dtype in_dtype, dn_dtype out_dtype,
                               hipStream_t stream) {
  return chunk_fwd_impl(q, k, v, nullptr, beta, S0, o, S_final, B, H, L, d_k, d_v, C, in_dtype,
                        out_dtype, nullptr, 0, stream, false, false, true);
}

int deltanet_gated_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const float* S0, void* o, float* S_final, int B,
                             int H, int L, int d_k, int d_v, int C, dn_dtype in_dtype, dn_dtype out_dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // With L = 0 there is no token to decay and alpha may be null: the call
  // only copies the state, as the plain forward does.
  if (L > 0 && !alpha) return DN_ERR_NULL_ARG;
  return chunk_fwd_impl(q, k, v, alpha, beta, S0, o, S_final, B, H, L, d_k, d_v, C, in_dtype,
                        out_dtype, workspace, workspace_bytes, stream);
}

int deltanet_decode_step(const void* q, const void* k, const void* v, const float* beta,
                         float* S, void* o, int B, int H, int d_k, int d_v, dn_dtype in_dtype,
                         dn_dtype out_dtype, hipStream_t stream) {
  return decode_impl(q, k, v, nullptr, beta, S, o, B, H, d_k, d_v, in_dtype, out_dtype, stream);
}

int deltanet_gated_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, float* S, void* o, int B, int H, int d_k,
                               int d_v, dn_dtype in_dtype, dn_dtype out_dtype, hipStream_t stream) {
  if (!alpha) return DN_ERR_NULL_ARG;
  return decode_impl(q, k, v, alpha, beta, S, o, B, H, d_k, d_v, in_dtype, out_dtype, stream);
}

}  // extern "C"
