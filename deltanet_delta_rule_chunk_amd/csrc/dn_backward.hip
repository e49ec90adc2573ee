// dn_backward.hip -- gradient of the chunked delta-rule forward: the fp32
// vector-ALU kernels (fp32 inputs) and the launch sequence; bf16 inputs run
// the matrix-core versions of the same five kernels (dn_backward_mfma.hip).
//
// The pages present the chunked form as the way to train the delta rule in
// linear time (page "GPT-2 から Kimi K3 まで、AI モデルの進化を解説", section
// "DeltaNet (Parallelizing linear transformers with delta rule)") without a
// backward pass; this one is derived from the chunk's forward by reverse-mode
// calculus.  Per chunk with entering state S, exit state S' and exit gradient
// G' = dL/dS':
//   forward:  A = tril(diag(beta) K K^T, -1), X = (I + A)^{-1},
//             T = X diag(beta), R = V - K S, Delta = T R,
//             M = tril(Q K^T) (diagonal included),
//             O = Q S + M Delta, S' = S + K^T Delta
//   backward: dDelta = M^T dO + K G',   dR = T^T dDelta,   dV = dR,
//             dS = G' + Q^T dO - K^T dR                   (the chunk's G)
//             dM = tril(dO Delta^T),    dQ = dO S^T + dM K,
//             dT = dDelta R^T,          dX = dT diag(beta),
//             dbeta_i += sum_r X_ri dT_ri,
//             dA = -X^T dX X^T (strictly lower),  W = diag(beta) dA,
//             dbeta_r += sum_{i<r} dA_ri (k_r . k_i),
//             dK = dM^T Q + Delta G'^T - dR S^T + W K + W^T K.
//
// Five launches, 64-row chunks (the chunk size does not change the result):
//   prep      (chunk, head): X and M;
//   fwd_scan  (head, 16 columns of d_v): the entering state S_c of every
//             chunk, R and Delta, into the workspace;
//   bwd_scan  (head, 16 columns), chunks in reverse: the exit gradient G'_c,
//             dDelta, dR (= dV, written out) and dS0;
//   cc_grad   (chunk, head): dM, dT, dA, W and dbeta;
//   qk_grad   (chunk, head): dQ and dK.
// (These are the fp32 path's kernels.  For bf16 inputs, dn_backward_mfma.hip
// has the prep of M and the last three on the matrix cores, and the
// chunked forward's own prep and scan at 128-token chunks stand in for the
// forward pass, writing X, S_c, R and Delta of every 64-row chunk.)
// A ragged last chunk reads zero rows (k = q = 0, beta = 0, dO = 0).

#include "dn_backward.h"
#include "dn_common.h"
#include "dn_launch.h"
#include "dn_valu_common.h"

namespace dn {
// The chunked forward's matrix-core kernels (dn_chunk_mfma.hip), which the
// bf16 backward runs as its forward pass.
size_t chunk_workspace_bytes_mfma(int B, int H, int L, int C);
hipError_t launch_chunk_fwd_mfma(const ChunkArgs& a);
}  // namespace dn

namespace dn {
namespace bwd {

using valu::load_rows;
constexpr int HV = 64;     // d_v columns staged at a time by the gradient kernels
constexpr int NTHR = 1024;
constexpr int LDC = C + 1;

// rows x cols of an fp32 matrix (row pitch src_ld) into LDS (row pitch ld);
// rows at or past rows_valid read as zero.
__device__ __forceinline__ void load_f32(float* dst, int ld, const float* src, int src_ld,
                                         int rows_valid, int rows, int cols) {
  for (int e = threadIdx.x; e < rows * cols; e += blockDim.x) {
    const int r = e / cols, c = e % cols;
    dst[r * ld + c] = r < rows_valid ? src[(size_t)r * src_ld + c] : 0.f;
  }
}

// A workgroup's ROWS x COLS tile held in registers, NTHR-strided (element
// e = threadIdx.x + p NTHR): the scans fetch the next chunk's operands into
// one while they compute the current chunk, then deposit it into LDS.
template <int ROWS, int COLS, typename T>
struct RegTile {
  static constexpr int N = ROWS * COLS / NTHR;
  static_assert(N * NTHR == ROWS * COLS, "tile");
  float x[N];
  __device__ __forceinline__ void load(const T* src, int rows_valid) {
#pragma unroll
    for (int p = 0; p < N; ++p) {
      const int e = threadIdx.x + p * NTHR, r = e / COLS;
      x[p] = r < rows_valid ? to_f32(src[e]) : 0.f;
    }
  }
  __device__ __forceinline__ void store(float* dst, int ld) const {
#pragma unroll
    for (int p = 0; p < N; ++p) {
      const int e = threadIdx.x + p * NTHR;
      dst[(e / COLS) * ld + e % COLS] = x[p];
    }
  }
};

// ---- prep: X = (I + A)^{-1} and M = tril(Q K^T) ---------------------------
template <int DK>
struct PrepSmem {
  static constexpr int LD = DK + 1;
  static constexpr size_t bytes = (2 * (size_t)C * LD + (size_t)C * LDC + C) * sizeof(float);
};

template <int DK, int DV, typename IT>
__global__ __launch_bounds__(NTHR) void prep_kernel(const IT* __restrict__ q,
                                                    const IT* __restrict__ k,
                                                    const float* __restrict__ beta, int L,
                                                    float* __restrict__ ws) {
  constexpr int LD = PrepSmem<DK>::LD;
  constexpr Ws W{DK, DV};
  extern __shared__ float smem[];
  float* Ks = smem;
  float* Qs = Ks + C * LD;   // Q, later X
  float* As = Qs + C * LD;
  float* bs = As + C * LDC;
  const int c = blockIdx.x, bh = blockIdx.y, nc = gridDim.x;
  const int valid = min(C, L - c * C);
  const size_t tok0 = (size_t)bh * L + (size_t)c * C;
  float* blk = ws + ((size_t)bh * nc + c) * W.per_chunk();

  load_rows(Ks, LD, k + tok0 * DK, valid, C, DK);
  load_rows(Qs, LD, q + tok0 * DK, valid, C, DK);
  for (int r = threadIdx.x; r < C; r += blockDim.x) bs[r] = r < valid ? beta[tok0 + r] : 0.f;
  __syncthreads();
  for (int e = threadIdx.x; e < C * C; e += blockDim.x) {
    const int r = e / C, i = e % C;
    float kk = 0.f, qk = 0.f;
    if (i <= r) {
      for (int d = 0; d < DK; ++d) {
        kk += Ks[r * LD + d] * Ks[i * LD + d];
        qk += Qs[r * LD + d] * Ks[i * LD + d];
      }
    }
    As[r * LDC + i] = i < r ? bs[r] * kk : 0.f;
    blk[W.M() + e] = qk;
  }
  valu::unit_lower_inverse<C>(As, LDC, Qs, LD);
  for (int e = threadIdx.x; e < C * C; e += blockDim.x) blk[W.X() + e] = Qs[(e / C) * LD + e % C];
}

// ---- fwd_scan: S_c, R, Delta ----------------------------------------------
template <int DK>
struct FwdSmem {
  static constexpr int LD = DK + 1;
  static constexpr size_t bytes =
      ((size_t)C * LD + (size_t)C * LDC + C + (size_t)DK * NT + 2 * (size_t)C * NT) * sizeof(float);
};

template <int DK, int DV, typename IT>
__global__ __launch_bounds__(NTHR) void fwd_scan_kernel(const IT* __restrict__ k,
                                                        const IT* __restrict__ v,
                                                        const float* __restrict__ beta,
                                                        const float* __restrict__ S0, int L,
                                                        int nc, float* __restrict__ ws) {
  constexpr int LD = FwdSmem<DK>::LD;
  constexpr Ws W{DK, DV};
  constexpr int RS = NTHR / NT;  // 64: one chunk row per thread
  constexpr int MS = DK / RS;    // state rows per thread
  static_assert(RS == C && MS * RS == DK, "thread map");
  extern __shared__ float smem[];
  float* Ks = smem;
  float* Xs = Ks + C * LD;
  float* bs = Xs + C * LDC;
  float* Ss = bs + C;
  float* Rs = Ss + DK * NT;
  float* Ds = Rs + C * NT;
  const int j0 = blockIdx.x * NT, bh = blockIdx.y;
  const int j = threadIdx.x % NT, r = threadIdx.x / NT;

  for (int m = 0; m < MS; ++m) {
    const int d = r + m * RS;
    Ss[d * NT + j] = S0 ? S0[((size_t)bh * DK + d) * DV + j0 + j] : 0.f;
  }
  RegTile<C, DK, IT> tk;
  RegTile<C, C, float> tx;
  float pb = 0.f, pv = 0.f;
  auto fetch = [&](int cc) {
    const int vc = min(C, L - cc * C);
    const size_t t0 = (size_t)bh * L + (size_t)cc * C;
    tk.load(k + t0 * DK, vc);
    tx.load(ws + ((size_t)bh * nc + cc) * W.per_chunk() + W.X(), C);
    pb = (int)threadIdx.x < vc ? beta[t0 + threadIdx.x] : 0.f;
    pv = r < vc ? to_f32(v[(t0 + r) * DV + j0 + j]) : 0.f;
  };
  if (nc > 0) fetch(0);
  for (int c = 0; c < nc; ++c) {
    float* blk = ws + ((size_t)bh * nc + c) * W.per_chunk();
    tk.store(Ks, LD);
    tx.store(Xs, LDC);
    if (threadIdx.x < C) bs[threadIdx.x] = pb;
    float acc = pv;
    __syncthreads();
    if (c + 1 < nc) fetch(c + 1);  // in flight while this chunk computes
    for (int m = 0; m < MS; ++m) {  // the entering state
      const int d = r + m * RS;
      blk[W.S() + (size_t)d * DV + j0 + j] = Ss[d * NT + j];
    }
    for (int d = 0; d < DK; ++d) acc -= Ks[r * LD + d] * Ss[d * NT + j];
    Rs[r * NT + j] = acc;
    blk[W.R() + (size_t)r * DV + j0 + j] = acc;
    __syncthreads();
    float dl = 0.f;
    for (int i = 0; i <= r; ++i) dl += Xs[r * LDC + i] * (bs[i] * Rs[i * NT + j]);
    Ds[r * NT + j] = dl;
    blk[W.D() + (size_t)r * DV + j0 + j] = dl;
    __syncthreads();
    for (int m = 0; m < MS; ++m) {
      const int d = r + m * RS;
      float s = Ss[d * NT + j];
      for (int i = 0; i < C; ++i) s += Ks[i * LD + d] * Ds[i * NT + j];
      Ss[d * NT + j] = s;
    }
    __syncthreads();
  }
}

// ---- bwd_scan: G'_c, dDelta, dR (= dV), dS0 -------------------------------
template <int DK>
struct BwdSmem {
  static constexpr int LD = DK + 1;
  static constexpr size_t bytes = (2 * (size_t)C * LD + 2 * (size_t)C * LDC + C +
                                   (size_t)DK * NT + 3 * (size_t)C * NT) * sizeof(float);
};

template <int DK, int DV, typename IT>
__global__ __launch_bounds__(NTHR) void bwd_scan_kernel(
    const IT* __restrict__ q, const IT* __restrict__ k, const float* __restrict__ beta,
    const float* __restrict__ dO, const float* __restrict__ dS_final, float* __restrict__ dv,
    float* __restrict__ dS0, int L, int nc, float* __restrict__ ws) {
  constexpr int LD = BwdSmem<DK>::LD;
  constexpr Ws W{DK, DV};
  constexpr int RS = NTHR / NT;
  constexpr int MS = DK / RS;
  static_assert(RS == C && MS * RS == DK, "thread map");
  extern __shared__ float smem[];
  float* Qs = smem;
  float* Ks = Qs + C * LD;
  float* Ms = Ks + C * LD;
  float* Xs = Ms + C * LDC;
  float* bs = Xs + C * LDC;
  float* Gs = bs + C;
  float* dOs = Gs + DK * NT;
  float* dDs = dOs + C * NT;
  float* dRs = dDs + C * NT;
  const int j0 = blockIdx.x * NT, bh = blockIdx.y;
  const int j = threadIdx.x % NT, r = threadIdx.x / NT;

  for (int m = 0; m < MS; ++m) {
    const int d = r + m * RS;
    Gs[d * NT + j] = dS_final ? dS_final[((size_t)bh * DK + d) * DV + j0 + j] : 0.f;
  }
  RegTile<C, DK, IT> tq, tk;
  RegTile<C, C, float> tm, tx;
  float pb = 0.f, pd = 0.f;
  auto fetch = [&](int cc) {
    const int vc = min(C, L - cc * C);
    const size_t t0 = (size_t)bh * L + (size_t)cc * C;
    const float* b = ws + ((size_t)bh * nc + cc) * W.per_chunk();
    tq.load(q + t0 * DK, vc);
    tk.load(k + t0 * DK, vc);
    tm.load(b + W.M(), C);
    tx.load(b + W.X(), C);
    pb = (int)threadIdx.x < vc ? beta[t0 + threadIdx.x] : 0.f;
    pd = r < vc ? dO[(t0 + r) * DV + j0 + j] : 0.f;
  };
  if (nc > 0) fetch(nc - 1);
  for (int c = nc - 1; c >= 0; --c) {
    const int valid = min(C, L - c * C);
    const size_t tok0 = (size_t)bh * L + (size_t)c * C;
    float* blk = ws + ((size_t)bh * nc + c) * W.per_chunk();
    tq.store(Qs, LD);
    tk.store(Ks, LD);
    tm.store(Ms, LDC);
    tx.store(Xs, LDC);
    if (threadIdx.x < C) bs[threadIdx.x] = pb;
    dOs[r * NT + j] = pd;
    __syncthreads();
    if (c > 0) fetch(c - 1);  // in flight while this chunk computes
    for (int m = 0; m < MS; ++m) {  // the exit gradient
      const int d = r + m * RS;
      blk[W.G() + (size_t)d * DV + j0 + j] = Gs[d * NT + j];
    }
    // dDelta_r = sum_{i >= r} M_ir dO_i + K_r G'
    float dd = 0.f;
    for (int i = r; i < C; ++i) dd += Ms[i * LDC + r] * dOs[i * NT + j];
    for (int d = 0; d < DK; ++d) dd += Ks[r * LD + d] * Gs[d * NT + j];
    dDs[r * NT + j] = dd;
    blk[W.dD() + (size_t)r * DV + j0 + j] = dd;
    __syncthreads();
    // dR_i = beta_i sum_{r >= i} X_ri dDelta_r  (row i = this thread's r)
    float dr = 0.f;
    for (int a = r; a < C; ++a) dr += Xs[a * LDC + r] * dDs[a * NT + j];
    dr *= bs[r];
    dRs[r * NT + j] = dr;
    if (r < valid) dv[(tok0 + r) * DV + j0 + j] = dr;
    __syncthreads();
    for (int m = 0; m < MS; ++m) {
      const int d = r + m * RS;
      float g = Gs[d * NT + j];
      for (int i = 0; i < C; ++i) g += Qs[i * LD + d] * dOs[i * NT + j] - Ks[i * LD + d] * dRs[i * NT + j];
      Gs[d * NT + j] = g;
    }
    __syncthreads();
  }
  if (dS0)
    for (int m = 0; m < MS; ++m) {
      const int d = r + m * RS;
      dS0[((size_t)bh * DK + d) * DV + j0 + j] = Gs[d * NT + j];
    }
}

// ---- cc_grad: dM, dT, dA, W, dbeta ----------------------------------------
template <int DK>
struct CcSmem {
  static constexpr int LD = DK + 1;
  static constexpr int LDH = HV + 1;
  static constexpr size_t bytes = (2 * (size_t)C * LDH + (size_t)C * LD + 4 * (size_t)C * LDC +
                                   2 * C) * sizeof(float);
};

template <int DK, int DV, typename IT>
__global__ __launch_bounds__(NTHR) void cc_grad_kernel(const IT* __restrict__ k,
                                                       const float* __restrict__ beta,
                                                       const float* __restrict__ dO,
                                                       float* __restrict__ dbeta, int L,
                                                       float* __restrict__ ws) {
  constexpr int LD = CcSmem<DK>::LD, LDH = CcSmem<DK>::LDH;
  constexpr Ws W{DK, DV};
  constexpr int PER = C * C / NTHR;  // C x C entries per thread
  constexpr int HW = DV < HV ? DV : HV;
  static_assert(PER * NTHR == C * C && DV % HW == 0, "shape");
  extern __shared__ float smem[];
  float* P1 = smem;
  float* P2 = P1 + C * LDH;
  float* Ks = P2 + C * LDH;
  float* Xs = Ks + C * LD;
  float* dMs = Xs + C * LDC;
  float* dTs = dMs + C * LDC;   // dT, then dX, then dA
  float* Ys = dTs + C * LDC;    // X^T dX
  float* bs = Ys + C * LDC;
  float* dbs = bs + C;
  const int c = blockIdx.x, bh = blockIdx.y, nc = gridDim.x;
  const int valid = min(C, L - c * C);
  const size_t tok0 = (size_t)bh * L + (size_t)c * C;
  float* blk = ws + ((size_t)bh * nc + c) * W.per_chunk();

  // dM = tril(dO Delta^T) and dT = dDelta R^T, over d_v in slices of HW.
  float am[PER], at[PER];
  for (int p = 0; p < PER; ++p) am[p] = at[p] = 0.f;
  for (int h = 0; h < DV; h += HW) {
    load_f32(P1, LDH, dO + tok0 * DV + h, DV, valid, C, HW);
    load_f32(P2, LDH, blk + W.D() + h, DV, C, C, HW);
    __syncthreads();
    {  // a thread's PER entries share the column i = threadIdx.x mod C
      const int i = threadIdx.x % C;
#pragma unroll 4
      for (int jj = 0; jj < HW; ++jj) {
        const float b = P2[i * LDH + jj];
#pragma unroll
        for (int p = 0; p < PER; ++p) am[p] += P1[((threadIdx.x + p * NTHR) / C) * LDH + jj] * b;
      }
    }
    __syncthreads();
    load_f32(P1, LDH, blk + W.dD() + h, DV, C, C, HW);
    load_f32(P2, LDH, blk + W.R() + h, DV, C, C, HW);
    __syncthreads();
    {  // a thread's PER entries share the column i = threadIdx.x mod C
      const int i = threadIdx.x % C;
#pragma unroll 4
      for (int jj = 0; jj < HW; ++jj) {
        const float b = P2[i * LDH + jj];
#pragma unroll
        for (int p = 0; p < PER; ++p) at[p] += P1[((threadIdx.x + p * NTHR) / C) * LDH + jj] * b;
      }
    }
    __syncthreads();
  }
  load_rows(Ks, LD, k + tok0 * DK, valid, C, DK);
  load_f32(Xs, LDC, blk + W.X(), C, C, C, C);
  for (int i = threadIdx.x; i < C; i += blockDim.x) bs[i] = i < valid ? beta[tok0 + i] : 0.f;
  for (int p = 0; p < PER; ++p) {
    const int e = threadIdx.x + p * NTHR, r = e / C, i = e % C;
    const float m_ = i <= r ? am[p] : 0.f, t_ = i <= r ? at[p] : 0.f;  // lower triangles
    dMs[r * LDC + i] = m_;
    dTs[r * LDC + i] = t_;
    blk[W.dM() + e] = m_;
  }
  __syncthreads();
  // dbeta_i from T = X diag(beta), then dX = dT diag(beta) in place.
  for (int i = threadIdx.x; i < C; i += blockDim.x) {
    float s = 0.f;
    for (int a = i; a < C; ++a) s += Xs[a * LDC + i] * dTs[a * LDC + i];
    dbs[i] = s;
  }
  __syncthreads();
  for (int p = 0; p < PER; ++p) {
    const int e = threadIdx.x + p * NTHR, r = e / C, i = e % C;
    dTs[r * LDC + i] *= bs[i];
  }
  __syncthreads();
  // Y = X^T dX (X and dX lower triangular: Y_ab sums over r >= max(a, b)).
  for (int p = 0; p < PER; ++p) {
    const int e = threadIdx.x + p * NTHR, a = e / C, b = e % C;
    float s = 0.f;
#pragma unroll 8
    for (int r = a > b ? a : b; r < C; ++r) s += Xs[r * LDC + a] * dTs[r * LDC + b];
    Ys[a * LDC + b] = s;
  }
  __syncthreads();
  // dA_ri = -sum_b Y_rb X_ib (b <= i) for i < r; W = diag(beta) dA.
  for (int p = 0; p < PER; ++p) {
    const int e = threadIdx.x + p * NTHR, r = e / C, i = e % C;
    float s = 0.f;
    if (i < r)
#pragma unroll 8
      for (int b = 0; b <= i; ++b) s -= Ys[r * LDC + b] * Xs[i * LDC + b];
    dTs[r * LDC + i] = s;
    blk[W.W() + e] = bs[r] * s;
  }
  __syncthreads();
  // dbeta_r += sum_{i < r} dA_ri (k_r . k_i): 16 lanes per row, then a
  // reduction across them.
  {
    const int r = threadIdx.x / 16, l = threadIdx.x % 16;
    float s = 0.f;
    for (int i = l; i < r; i += 16) {
      float kk = 0.f;
#pragma unroll 8
      for (int d = 0; d < DK; ++d) kk += Ks[r * LD + d] * Ks[i * LD + d];
      s += dTs[r * LDC + i] * kk;
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (l == 0 && r < valid) dbeta[tok0 + r] = dbs[r] + s;
  }
}

// ---- qk_grad: dQ, dK --------------------------------------------------------
template <int DK>
struct QkSmem {
  static constexpr int LD = DK + 1;
  static constexpr int LDH = HV + 1;
  static constexpr size_t phase1 = 2 * (size_t)DK * LDH + 3 * (size_t)C * LDH;
  static constexpr size_t phase2 = 2 * (size_t)C * LD + 2 * (size_t)C * LDC;
  static constexpr size_t bytes = (phase1 > phase2 ? phase1 : phase2) * sizeof(float);
};

template <int DK, int DV, typename IT>
__global__ __launch_bounds__(NTHR) void qk_grad_kernel(
    const IT* __restrict__ q, const IT* __restrict__ k, const float* __restrict__ dO,
    const float* __restrict__ dv, float* __restrict__ dq, float* __restrict__ dk, int L,
    const float* __restrict__ ws) {
  constexpr int LD = QkSmem<DK>::LD, LDH = QkSmem<DK>::LDH;
  constexpr Ws W{DK, DV};
  constexpr int HW = DV < HV ? DV : HV;
  constexpr int NCG = NTHR / C;   // 16 column groups
  constexpr int MC = DK / NCG;    // columns per thread
  static_assert(MC * NCG == DK, "thread map");
  extern __shared__ float smem[];
  const int c = blockIdx.x, bh = blockIdx.y, nc = gridDim.x;
  const int valid = min(C, L - c * C);
  const size_t tok0 = (size_t)bh * L + (size_t)c * C;
  const float* blk = ws + ((size_t)bh * nc + c) * W.per_chunk();
  const int r = threadIdx.x / NCG, cg = threadIdx.x % NCG;

  float aq[MC], ak[MC];
  for (int m = 0; m < MC; ++m) aq[m] = ak[m] = 0.f;
  {  // dO S^T, Delta G'^T - dR S^T over d_v in slices
    float* Sh = smem;
    float* Gh = Sh + DK * LDH;
    float* dOh = Gh + DK * LDH;
    float* Dh = dOh + C * LDH;
    float* dRh = Dh + C * LDH;
    for (int h = 0; h < DV; h += HW) {
      load_f32(Sh, LDH, blk + W.S() + h, DV, DK, DK, HW);
      load_f32(Gh, LDH, blk + W.G() + h, DV, DK, DK, HW);
      load_f32(dOh, LDH, dO + tok0 * DV + h, DV, valid, C, HW);
      load_f32(Dh, LDH, blk + W.D() + h, DV, C, C, HW);
      load_f32(dRh, LDH, dv + tok0 * DV + h, DV, valid, C, HW);
      __syncthreads();
      // One read of this row's dO, Delta, dR per column feeds all MC outputs.
#pragma unroll 2
      for (int jj = 0; jj < HW; ++jj) {
        const float o_ = dOh[r * LDH + jj], dl = Dh[r * LDH + jj], rr = dRh[r * LDH + jj];
#pragma unroll
        for (int m = 0; m < MC; ++m) {
          const int d = cg + m * NCG;
          const float sv = Sh[d * LDH + jj];
          aq[m] += o_ * sv;
          ak[m] += dl * Gh[d * LDH + jj] - rr * sv;
        }
      }
      __syncthreads();
    }
  }
  {  // dM K; dM^T Q + W K + W^T K
    float* Qs = smem;
    float* Ks = Qs + C * LD;
    float* dMs = Ks + C * LD;
    float* Wm = dMs + C * LDC;
    load_rows(Qs, LD, q + tok0 * DK, valid, C, DK);
    load_rows(Ks, LD, k + tok0 * DK, valid, C, DK);
    load_f32(dMs, LDC, blk + W.dM(), C, C, C, C);
    load_f32(Wm, LDC, blk + W.W(), C, C, C, C);
    __syncthreads();
    // dM and W hold zeros outside their triangles, so every row a can be
    // summed: dM_ra (a <= r), dM_ar (a >= r), W_ra + W_ar.
#pragma unroll 2
    for (int a = 0; a < C; ++a) {
      const float mra = dMs[r * LDC + a], mar = dMs[a * LDC + r];
      const float w = Wm[r * LDC + a] + Wm[a * LDC + r];
#pragma unroll
      for (int m = 0; m < MC; ++m) {
        const int d = cg + m * NCG;
        const float kv = Ks[a * LD + d];
        aq[m] += mra * kv;
        ak[m] += mar * Qs[a * LD + d] + w * kv;
      }
    }
  }
  if (r < valid)
    for (int m = 0; m < MC; ++m) {
      const int d = cg + m * NCG;
      dq[(tok0 + r) * DK + d] = aq[m];
      dk[(tok0 + r) * DK + d] = ak[m];
    }
}

template <typename K>
static hipError_t set_smem(K* kernel, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

#define DN_TRY(x)                      \
  do {                                 \
    hipError_t e_ = (x);               \
    if (e_ != hipSuccess) return e_;   \
  } while (0)

template <int DK, int DV, typename IT>
hipError_t launch_t(const BwdArgs& a) {
  const int nc = cdiv(a.L, C);
  const int bh = a.B * a.H;
  float* ws = static_cast<float*>(a.workspace);
  const IT *q = static_cast<const IT*>(a.q), *k = static_cast<const IT*>(a.k);
  const IT* v = static_cast<const IT*>(a.v);
  const dim3 chunks(nc, bh), slices(DV / NT, bh), blk(NTHR);
  // bf16 q, k, v: the five kernels' products run on the matrix cores
  // (dn_backward_mfma.hip); fp32 inputs keep the vector-ALU kernels below.
  constexpr bool kMatrixCores = sizeof(IT) == 2;
  if (nc > 0) {
    prof_mark(kSlotBwdPrep, false, a.stream);
    if constexpr (kMatrixCores) {
      DN_TRY(launch_prep_mfma(DK, DV, q, k, a.L, nc, bh, ws, a.stream));
    } else {
      DN_TRY(set_smem(&prep_kernel<DK, DV, IT>, PrepSmem<DK>::bytes));
      hipLaunchKernelGGL((prep_kernel<DK, DV, IT>), chunks, blk, PrepSmem<DK>::bytes, a.stream, q,
                         k, a.beta, a.L, ws);
      DN_TRY(hipGetLastError());
    }
    prof_mark(kSlotBwdPrep, true, a.stream);
    prof_mark(kSlotBwdFwdScan, false, a.stream);
    if constexpr (kMatrixCores) {
      // The forward pass on the chunked forward's kernels at 128-token
      // chunks (their T in the workspace past the 64-token blocks), writing
      // X, S, R and Delta of every 64-token block.
      constexpr Ws W{DK, DV};
      const BwdFwdOut bo{ws, W.per_chunk(), W.X(), W.S(), W.R(), W.D(), nc};
      ChunkArgs ca{k, k, v, nullptr, a.beta, a.S0, nullptr, nullptr, a.B, a.H, a.L, DK, DV, 128,
                   1, 0, ws + (size_t)bh * nc * W.per_chunk(), a.stream, false};
      ca.bwd_out = &bo;
      DN_TRY(launch_chunk_fwd_mfma(ca));
    } else {
      DN_TRY(set_smem(&fwd_scan_kernel<DK, DV, IT>, FwdSmem<DK>::bytes));
      hipLaunchKernelGGL((fwd_scan_kernel<DK, DV, IT>), slices, blk, FwdSmem<DK>::bytes, a.stream,
                         k, v, a.beta, a.S0, a.L, nc, ws);
      DN_TRY(hipGetLastError());
    }
    prof_mark(kSlotBwdFwdScan, true, a.stream);
  }
  prof_mark(kSlotBwdScan, false, a.stream);
  if (kMatrixCores && nc > 0) {
    DN_TRY(launch_bwd_scan_mfma(DK, DV, q, k, a.beta, a.dO, a.dS_final, a.dv, a.dS0, a.L, nc, bh,
                                ws, a.stream));
  } else {
    DN_TRY(set_smem(&bwd_scan_kernel<DK, DV, IT>, BwdSmem<DK>::bytes));
    hipLaunchKernelGGL((bwd_scan_kernel<DK, DV, IT>), slices, blk, BwdSmem<DK>::bytes, a.stream, q,
                       k, a.beta, a.dO, a.dS_final, a.dv, a.dS0, a.L, nc, ws);
    DN_TRY(hipGetLastError());
  }
  prof_mark(kSlotBwdScan, true, a.stream);
  if (nc > 0) {
    if constexpr (kMatrixCores) {
      // One kernel for the C x C gradients and dQ, dK (profiled as the latter).
      prof_mark(kSlotBwdQk, false, a.stream);
      DN_TRY(launch_grad_mfma(DK, DV, q, k, a.beta, a.dO, a.dv, a.dq, a.dk, a.dbeta, a.L, nc, bh,
                              ws, a.stream));
      prof_mark(kSlotBwdQk, true, a.stream);
    } else {
      prof_mark(kSlotBwdCc, false, a.stream);
      DN_TRY(set_smem(&cc_grad_kernel<DK, DV, IT>, CcSmem<DK>::bytes));
      hipLaunchKernelGGL((cc_grad_kernel<DK, DV, IT>), chunks, blk, CcSmem<DK>::bytes, a.stream, k,
                         a.beta, a.dO, a.dbeta, a.L, ws);
      DN_TRY(hipGetLastError());
      prof_mark(kSlotBwdCc, true, a.stream);
      prof_mark(kSlotBwdQk, false, a.stream);
      DN_TRY(set_smem(&qk_grad_kernel<DK, DV, IT>, QkSmem<DK>::bytes));
      hipLaunchKernelGGL((qk_grad_kernel<DK, DV, IT>), chunks, blk, QkSmem<DK>::bytes, a.stream, q,
                         k, a.dO, a.dv, a.dq, a.dk, a.L, ws);
      DN_TRY(hipGetLastError());
      prof_mark(kSlotBwdQk, true, a.stream);
    }
  }
  return hipSuccess;
}
#undef DN_TRY

template <int DK, int DV>
hipError_t launch_types(const BwdArgs& a) {
  return a.in_dtype == 1 ? launch_t<DK, DV, bf16>(a) : launch_t<DK, DV, float>(a);
}

}  // namespace bwd

size_t chunk_bwd_workspace_bytes(int B, int H, int L, int d_k, int d_v) {
  // The 64-token blocks, then the T fragments of the forward pass at
  // 128-token chunks (bf16 path).
  return (size_t)B * H * cdiv(L, bwd::C) * bwd::Ws{d_k, d_v}.per_chunk() * sizeof(float) +
         chunk_workspace_bytes_mfma(B, H, L, 128);
}

hipError_t launch_chunk_bwd(const BwdArgs& a) {
  if (a.d_k == 64 && a.d_v == 64) return bwd::launch_types<64, 64>(a);
  if (a.d_k == 64 && a.d_v == 128) return bwd::launch_types<64, 128>(a);
  if (a.d_k == 128 && a.d_v == 64) return bwd::launch_types<128, 64>(a);
  return bwd::launch_types<128, 128>(a);
}

}  // namespace dn
