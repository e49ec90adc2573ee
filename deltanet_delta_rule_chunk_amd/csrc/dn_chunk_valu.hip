// dn_chunk_valu.hip -- chunkwise-parallel delta-rule forward, fp32 vector-ALU
// kernels.  This is the path for fp32 inputs (and any shape the matrix-core
// path does not cover); all arithmetic is fp32.
//
// The chunked form (page "GPT-2 から Kimi K3 まで、AI モデルの進化を解説",
// section "DeltaNet (Parallelizing linear transformers with delta rule)":
// each chunk's outputs follow from the previous chunk's final state and the
// chunk's own q, k, v, via generalised-Householder transitions).  Written out
// from the recurrence, for a chunk with rows K, Q, V, beta and entering state S:
//     A     = tril(diag(beta) K K^T, -1)
//     T     = (I + A)^{-1} diag(beta)                (lower triangular)
//     Delta = T (V - K S)
//     O     = Q S + tril(Q K^T) Delta                (diagonal included)
//     S'    = S + K^T Delta
// Two launches:
//   prep  (one workgroup per chunk, all chunks in parallel): T and
//         P = tril(Q K^T) into the workspace;
//   scan  (one workgroup per (head, 16-column slice of d_v)): walks the
//         chunks in order with the state slice resident in LDS.  The columns
//         of S evolve independently (every product above acts on S from the
//         left), so slices of d_v are independent scans.
// A ragged last chunk reads k = q = v = 0 and beta = 0 past L: zero rows of K
// and beta make those rows of T, Delta and every state contribution zero.
//
// Gated form (GATED = true; Gated DeltaNet, article "How a Baseten Engineer
// Traced 7 Years of Attention Mechanism Evolution", Gated DeltaNet section:
// decay the state by alpha_t, then the precise write).  With the within-chunk
// cumulative log-decays g_r = sum_{j<=r} log alpha_j (rows past L: alpha = 1)
// and E_ri = e^{g_r - g_i} (i <= r, so every factor is <= 1):
//     A     = tril(diag(beta) (K K^T o E), -1)
//     Delta = T (V - diag(e^g) K S)
//     O     = diag(e^g) Q S + (tril(Q K^T) o E) Delta
//     S'    = e^{g_C} S + K^T diag(e^{g_C - g}) Delta
// (o = elementwise product).  The prep kernel writes g next to T and P.

#include "dn_common.h"
#include "dn_launch.h"
#include "dn_valu_common.h"

namespace dn {
namespace valu {

constexpr int NT = 16;  // d_v columns per scan workgroup

template <int C, int DK>
struct PrepSmem {
  static constexpr int LD = (C > DK ? C : DK) + 1;  // row pitch in floats
  static constexpr size_t bytes = 2 * (size_t)C * LD * sizeof(float) + 2 * C * sizeof(float);
};


// One workgroup per (chunk, head).  Writes T[C][C] and P[C][C] (fp32, full
// squares with zeros above the diagonal) for the chunk.
template <int C, int DK, typename IT, bool GATED>
__global__ __launch_bounds__(256) void prep_kernel(const IT* __restrict__ q,
                                                   const IT* __restrict__ k,
                                                   const float* __restrict__ alpha,
                                                   const float* __restrict__ beta, int L,
                                                   float* __restrict__ Tws,
                                                   float* __restrict__ Pws,
                                                   float* __restrict__ Gws) {
  constexpr int LD = PrepSmem<C, DK>::LD;
  extern __shared__ float smem[];
  float* buf0 = smem;
  float* buf1 = smem + C * LD;
  float* bs = smem + 2 * C * LD;
  float* gs = bs + C;  // within-chunk cumulative log-decays (gated form)

  const int c = blockIdx.x, bh = blockIdx.y, nc = gridDim.x;
  const int t0 = c * C;
  const int valid = min(C, L - t0);
  const size_t tok0 = (size_t)bh * L + t0;
  float* Tc = Tws + ((size_t)bh * nc + c) * C * C;
  float* Pc = Pws + ((size_t)bh * nc + c) * C * C;

  load_rows(buf0, LD, k + tok0 * DK, valid, C, DK);
  for (int r = threadIdx.x; r < C; r += blockDim.x) bs[r] = r < valid ? beta[tok0 + r] : 0.f;
  if constexpr (GATED) {
    for (int r = threadIdx.x; r < C; r += blockDim.x) gs[r] = r < valid ? log_decay(alpha[tok0 + r]) : 0.f;
    __syncthreads();
    if (threadIdx.x == 0) {  // prefix sum, in row order
      float acc = 0.f;
      for (int r = 0; r < C; ++r) gs[r] = acc += gs[r];
    }
    __syncthreads();
    for (int r = threadIdx.x; r < C; r += blockDim.x) Gws[((size_t)bh * nc + c) * C + r] = gs[r];
  }
  __syncthreads();

  // A = tril(diag(beta) (K K^T o E), -1) into buf1.
  for (int e = threadIdx.x; e < C * C; e += blockDim.x) {
    const int r = e / C, i = e % C;
    float acc = 0.f;
    if (i < r) {
      for (int d = 0; d < DK; ++d) acc += buf0[r * LD + d] * buf0[i * LD + d];
      acc *= bs[r];
      if constexpr (GATED) acc *= expf(gs[r] - gs[i]);
    }
    buf1[r * LD + i] = acc;
  }
  __syncthreads();

  // X = (I + A)^{-1} into buf0.
  unit_lower_inverse<C>(buf1, LD, buf0, LD);

  // T = X diag(beta).
  for (int e = threadIdx.x; e < C * C; e += blockDim.x) {
    const int r = e / C, i = e % C;
    Tc[e] = buf0[r * LD + i] * bs[i];
  }
  __syncthreads();

  // P = tril(Q K^T) (o E in the gated form), diagonal included.
  load_rows(buf1, LD, k + tok0 * DK, valid, C, DK);
  load_rows(buf0, LD, q + tok0 * DK, valid, C, DK);
  __syncthreads();
  for (int e = threadIdx.x; e < C * C; e += blockDim.x) {
    const int r = e / C, i = e % C;
    float acc = 0.f;
    if (i <= r) {
      for (int d = 0; d < DK; ++d) acc += buf0[r * LD + d] * buf1[i * LD + d];
      if constexpr (GATED) acc *= expf(gs[r] - gs[i]);
    }
    Pc[e] = acc;
  }
}

template <int C, int DK>
struct ScanSmem {
  static constexpr int LDK = DK + 1;
  static constexpr size_t bytes =
      ((size_t)C * LDK + (size_t)DK * NT + 2 * (size_t)C * NT + C) * sizeof(float);
};

// One workgroup per (16-column slice of d_v, head).  Walks all chunks.
template <int C, int DK, int DV, typename IT, typename OT, bool GATED>
__global__ __launch_bounds__(256) void scan_kernel(
    const IT* __restrict__ q, const IT* __restrict__ k, const IT* __restrict__ v,
    const float* __restrict__ S0, OT* __restrict__ o, float* __restrict__ S_final, int L,
    int nc, const float* __restrict__ Tws, const float* __restrict__ Pws,
    const float* __restrict__ Gws) {
  constexpr int LDK = ScanSmem<C, DK>::LDK;
  constexpr int RSTRIDE = 256 / NT;   // rows between a thread's outputs
  constexpr int MR = C / RSTRIDE;     // chunk rows per thread
  constexpr int MS = DK / RSTRIDE;    // state rows per thread
  extern __shared__ float smem[];
  float* Ks = smem;
  float* Ss = Ks + C * LDK;
  float* Rs = Ss + DK * NT;
  float* Ds = Rs + C * NT;
  float* gs = Ds + C * NT;  // the chunk's cumulative log-decays (gated form)

  const int j0 = blockIdx.x * NT, bh = blockIdx.y;
  const int j = threadIdx.x % NT, rb = threadIdx.x / NT;
  const size_t sbase = (size_t)bh * DK * DV;

  for (int m = 0; m < MS; ++m) {
    const int d = rb + m * RSTRIDE;
    Ss[d * NT + j] = S0 ? S0[sbase + (size_t)d * DV + j0 + j] : 0.f;
  }

  for (int c = 0; c < nc; ++c) {
    const int t0 = c * C;
    const int valid = min(C, L - t0);
    const size_t tok0 = (size_t)bh * L + t0;
    const float* Tc = Tws + ((size_t)bh * nc + c) * C * C;
    const float* Pc = Pws + ((size_t)bh * nc + c) * C * C;
    load_rows(Ks, LDK, k + tok0 * DK, valid, C, DK);
    if constexpr (GATED)
      for (int r = threadIdx.x; r < C; r += blockDim.x) gs[r] = Gws[((size_t)bh * nc + c) * C + r];
    __syncthreads();

    // R = V - K S into LDS; O_inter = Q S kept in registers (each row scaled
    // by e^{g_r} in the gated form).
    float oi[MR];
    for (int m = 0; m < MR; ++m) {
      const int r = rb + m * RSTRIDE;
      float ks = 0.f, qs = 0.f;
      if (r < valid) {
        const IT* qr = q + (tok0 + r) * DK;
#pragma unroll 8
        for (int d = 0; d < DK; ++d) {
          const float sd = Ss[d * NT + j];
          ks += Ks[r * LDK + d] * sd;
          qs += to_f32(qr[d]) * sd;
        }
      }
      const float vr = r < valid ? to_f32(v[(tok0 + r) * DV + j0 + j]) : 0.f;
      if constexpr (GATED) {
        const float dr = expf(gs[r]);
        ks *= dr;
        qs *= dr;
      }
      Rs[r * NT + j] = vr - ks;
      oi[m] = qs;
    }
    __syncthreads();

    // Delta = T R.
    for (int m = 0; m < MR; ++m) {
      const int r = rb + m * RSTRIDE;
      float acc = 0.f;
#pragma unroll 8
      for (int i = 0; i <= r; ++i) acc += Tc[r * C + i] * Rs[i * NT + j];
      Ds[r * NT + j] = acc;
    }
    __syncthreads();

    // O = O_inter + P Delta.
    for (int m = 0; m < MR; ++m) {
      const int r = rb + m * RSTRIDE;
      if (r < valid) {
        float acc = oi[m];
#pragma unroll 8
        for (int i = 0; i <= r; ++i) acc += Pc[r * C + i] * Ds[i * NT + j];
        o[(tok0 + r) * DV + j0 + j] = from_f32<OT>(acc);
      }
    }

    // S += K^T Delta  (gated: S = e^{g_C} S + K^T diag(e^{g_C - g}) Delta).
    for (int m = 0; m < MS; ++m) {
      const int d = rb + m * RSTRIDE;
      float acc = Ss[d * NT + j];
      if constexpr (GATED) {
        const float gC = gs[C - 1];
        acc *= expf(gC);
#pragma unroll 8
        for (int r = 0; r < C; ++r) acc += Ks[r * LDK + d] * (expf(gC - gs[r]) * Ds[r * NT + j]);
      } else {
#pragma unroll 8
        for (int r = 0; r < C; ++r) acc += Ks[r * LDK + d] * Ds[r * NT + j];
      }
      Ss[d * NT + j] = acc;
    }
    __syncthreads();
  }

  if (S_final) {
    __syncthreads();
    for (int m = 0; m < MS; ++m) {
      const int d = rb + m * RSTRIDE;
      S_final[sbase + (size_t)d * DV + j0 + j] = Ss[d * NT + j];
    }
  }
}

template <int C, int DK, int DV, typename IT, typename OT, bool GATED>
hipError_t launch_t(const ChunkArgs& a) {
  const int nc = cdiv(a.L, C);
  const int bh = a.B * a.H;
  float* Tws = static_cast<float*>(a.workspace);
  float* Pws = Tws + (size_t)bh * nc * C * C;
  float* Gws = Pws + (size_t)bh * nc * C * C;  // gated form only
  if (nc > 0) {
    constexpr size_t sm = PrepSmem<C, DK>::bytes;
    hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&prep_kernel<C, DK, IT, GATED>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    if (e != hipSuccess) return e;
    prof_mark(kSlotChunkPrep, false, a.stream);
    hipLaunchKernelGGL((prep_kernel<C, DK, IT, GATED>), dim3(nc, bh), dim3(256), sm, a.stream,
                       static_cast<const IT*>(a.q), static_cast<const IT*>(a.k), a.alpha,
                       a.beta, a.L, Tws, Pws, Gws);
    e = hipGetLastError();
    prof_mark(kSlotChunkPrep, true, a.stream);
    if (e != hipSuccess) return e;
  }
  constexpr size_t sm2 = ScanSmem<C, DK>::bytes;
  hipError_t e =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_kernel<C, DK, DV, IT, OT, GATED>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm2);
  if (e != hipSuccess) return e;
  prof_mark(kSlotChunkScan, false, a.stream);
  hipLaunchKernelGGL((scan_kernel<C, DK, DV, IT, OT, GATED>), dim3(DV / NT, bh), dim3(256), sm2,
                     a.stream, static_cast<const IT*>(a.q), static_cast<const IT*>(a.k),
                     static_cast<const IT*>(a.v), a.S0, static_cast<OT*>(a.o), a.S_final, a.L,
                     nc, Tws, Pws, Gws);
  e = hipGetLastError();
  prof_mark(kSlotChunkScan, true, a.stream);
  return e;
}

template <int C, int DK, int DV, typename IT, typename OT>
hipError_t launch_g(const ChunkArgs& a) {
  return a.alpha ? launch_t<C, DK, DV, IT, OT, true>(a) : launch_t<C, DK, DV, IT, OT, false>(a);
}

template <int C, int DK, int DV>
hipError_t launch_types(const ChunkArgs& a) {
  if (a.in_dtype == 0 && a.out_dtype == 0) return launch_g<C, DK, DV, float, float>(a);
  if (a.in_dtype == 0 && a.out_dtype == 1) return launch_g<C, DK, DV, float, bf16>(a);
  if (a.in_dtype == 1 && a.out_dtype == 0) return launch_g<C, DK, DV, bf16, float>(a);
  return launch_g<C, DK, DV, bf16, bf16>(a);
}

template <int C>
hipError_t launch_c(const ChunkArgs& a) {
  if (a.d_k == 64 && a.d_v == 64) return launch_types<C, 64, 64>(a);
  if (a.d_k == 64 && a.d_v == 128) return launch_types<C, 64, 128>(a);
  if (a.d_k == 128 && a.d_v == 64) return launch_types<C, 128, 64>(a);
  return launch_types<C, 128, 128>(a);
}

}  // namespace valu

size_t chunk_workspace_bytes_valu(int B, int H, int L, int C) {
  const size_t nc = (size_t)cdiv(L, C);
  return 2 * (size_t)B * H * nc * C * C * sizeof(float);
}

hipError_t launch_chunk_fwd_valu(const ChunkArgs& a) {
  return a.C == 64 ? valu::launch_c<64>(a) : valu::launch_c<128>(a);
}

}  // namespace dn
