// dn_kda.hip -- chunked delta rule with per-dimension decay (KDA), fp32
// vector-ALU kernels.
//
// The article "How a Baseten Engineer Traced 7 Years of Attention Mechanism
// Evolution" (wpnews.pro / dev.to) describes Kimi Linear's KDA as Gated
// DeltaNet with its scalar gate turned into a vector: every dimension of the
// memory forgets at its own rate.  With S a d_k x d_v state read as
// v_old = k S, per token: S <- diag(alpha_t) S, then the delta write on the
// decayed state (u_t = beta_t (v_t - k_t S), S <- S + k_t^T u_t), o_t = q_t S.
//
// Chunked form, written out from that recurrence.  Within a chunk let g_r be
// the d_k-vector of cumulative log-decays, g_r = log(alpha_1) + ... +
// log(alpha_r) (per dimension; rows past L: alpha = 1).  Unrolling the chunk
// from its entering state S gives, with every exponent <= 0,
//     A_ri  = beta_r sum_j k_rj k_ij e^{g_rj - g_ij}       (i < r)
//     T     = (I + A)^{-1} diag(beta)
//     Delta = T (V - (K o e^g) S)
//     P_ri  = sum_j q_rj k_ij e^{g_rj - g_ij}              (i <= r)
//     O     = (Q o e^g) S + P Delta
//     S'    = diag(e^{g_C}) S + (K o e^{g_C - g})^T Delta
// (o: elementwise, row by row).  Unlike the scalar gate, the pair factors
// e^{g_r - g_i} differ per dimension, so they do not factor into matrix-core
// operands with bounded exponents (K o e^{-g} grows without bound along the
// chunk); these kernels take them elementwise in fp32.
//
// Two launches, 64-row chunks (the result does not depend on the chunk
// size, so the C the caller names is not used):
//   prep (one workgroup per (chunk, head), all in parallel): g by a prefix
//        sum per dimension, then T, P and the decayed operands
//        K o e^g, Q o e^g, K o e^{g_C - g} and e^{g_C} into the workspace;
//   scan (one workgroup per (head, 16 columns of d_v)): walks the chunks in
//        order with its state columns in LDS (the columns of S evolve
//        independently), staging each chunk's operands into LDS first.

#include "dn_common.h"
#include "dn_kda.h"
#include "dn_launch.h"
#include "dn_valu_common.h"

namespace dn {
namespace kda {

using valu::load_rows;
constexpr int NTHR = 1024; // threads per workgroup: the LDS a chunk needs
                           // allows one workgroup per CU, so it brings 16
                           // waves to hide LDS and memory latency

template <int DK>
struct PrepSmem {
  static constexpr int LD = DK + 1;  // row pitch of the C x d_k tiles
  static constexpr int LDA = C + 1;  // row pitch of A
  static constexpr size_t floats = 3 * (size_t)C * LD + (size_t)C * LDA + C;
  static constexpr size_t bytes = floats * sizeof(float);
};

template <int DK, typename IT>
__global__ __launch_bounds__(NTHR) void prep_kernel(const IT* __restrict__ q,
                                                   const IT* __restrict__ k,
                                                   const float* __restrict__ alpha,
                                                   const float* __restrict__ beta, int L,
                                                   float* __restrict__ ws) {
  constexpr int LD = PrepSmem<DK>::LD, LDA = PrepSmem<DK>::LDA;
  extern __shared__ float smem[];
  float* Ks = smem;            // K, later X = (I + A)^{-1}
  float* Qs = Ks + C * LD;     // Q
  float* Gs = Qs + C * LD;     // g (cumulative log-decays)
  float* As = Gs + C * LD;     // A
  float* bs = As + C * LDA;    // beta

  const int c = blockIdx.x, bh = blockIdx.y, nc = gridDim.x;
  const int t0 = c * C;
  const int valid = min(C, L - t0);
  const size_t tok0 = (size_t)bh * L + t0;
  float* Tc = ws + ((size_t)bh * nc + c) * chunk_floats(DK);
  float* Pc = Tc + C * C;
  float* Kd = Pc + C * C;    // K o e^g
  float* Qd = Kd + C * DK;   // Q o e^g
  float* Ku = Qd + C * DK;   // K o e^{g_C - g}
  float* gam = Ku + C * DK;  // e^{g_C}

  load_rows(Ks, LD, k + tok0 * DK, valid, C, DK);
  load_rows(Qs, LD, q + tok0 * DK, valid, C, DK);
  for (int r = threadIdx.x; r < C; r += blockDim.x) bs[r] = r < valid ? beta[tok0 + r] : 0.f;
  // g: the log-decays of the whole tile at once (coalesced), then a prefix
  // sum down each dimension's column (rows past L add zero): 8 segments of 8
  // rows per column, each summed in registers, then offset by the totals of
  // the segments above it (parked in the A tile, which is written only later).
  for (int e = threadIdx.x; e < C * DK; e += blockDim.x) {
    const int r = e / DK, j = e % DK;
    Gs[r * LD + j] = r < valid ? log_decay(alpha[(tok0 + r) * DK + j]) : 0.f;
  }
  __syncthreads();
  {
    static_assert(8 * DK <= NTHR && 8 * DK <= C * LDA && C == 64, "prefix layout");
    const int j = threadIdx.x % DK, seg = threadIdx.x / DK;
    float v[8];
    if (seg < 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = Gs[(8 * seg + i) * LD + j];
#pragma unroll
      for (int i = 1; i < 8; ++i) v[i] += v[i - 1];
      As[seg * DK + j] = v[7];
    }
    __syncthreads();
    if (seg < 8) {
      float off = 0.f;
      for (int s2 = 0; s2 < seg; ++s2) off += As[s2 * DK + j];
#pragma unroll
      for (int i = 0; i < 8; ++i) Gs[(8 * seg + i) * LD + j] = v[i] + off;
    }
  }
  __syncthreads();

  // The decayed operands of the scan.
  for (int e = threadIdx.x; e < C * DK; e += blockDim.x) {
    const int r = e / DK, j = e % DK;
    const float g = Gs[r * LD + j], gC = Gs[(C - 1) * LD + j];
    const float kv = Ks[r * LD + j];
    Kd[e] = kv * __expf(g);
    Qd[e] = Qs[r * LD + j] * __expf(g);
    Ku[e] = kv * __expf(gC - g);
  }
  for (int j = threadIdx.x; j < DK; j += blockDim.x) gam[j] = __expf(Gs[(C - 1) * LD + j]);

  // A (strictly lower) into LDS and P (lower, diagonal included) to the
  // workspace; both share the factors e^{g_rj - g_ij} <= 1.
  for (int e = threadIdx.x; e < C * C; e += blockDim.x) {
    const int r = e / C, i = e % C;
    float a = 0.f, p = 0.f;
    if (i <= r) {
      const float *kr = Ks + r * LD, *ki = Ks + i * LD, *qr = Qs + r * LD;
      const float *gr = Gs + r * LD, *gi = Gs + i * LD;
      for (int j = 0; j < DK; ++j) {
        const float f = __expf(gr[j] - gi[j]) * ki[j];
        a += kr[j] * f;
        p += qr[j] * f;
      }
    }
    As[r * LDA + i] = i < r ? a * bs[r] : 0.f;
    Pc[e] = p;
  }

  // X = (I + A)^{-1} over the K tile (no longer needed), then T = X diag(beta).
  valu::unit_lower_inverse<C>(As, LDA, Ks, LD);
  for (int e = threadIdx.x; e < C * C; e += blockDim.x) {
    const int r = e / C, i = e % C;
    Tc[e] = Ks[r * LD + i] * bs[i];
  }
}

template <int DK>
struct ScanSmem {
  static constexpr int LDK = DK + 1;  // row pitch of the C x d_k tiles
  static constexpr int LDC = C + 1;   // row pitch of T and P
  static constexpr size_t floats = 3 * (size_t)C * LDK + 2 * (size_t)C * LDC + (size_t)DK * NT +
                                   2 * (size_t)C * NT + DK;
  static constexpr size_t bytes = floats * sizeof(float);
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

// One workgroup per (16-column slice of d_v, head).  Walks all chunks.  Each
// chunk's workspace block (T, P, the three decayed tiles, e^{g_C}: 145 KB
// at d_k = 128) is contiguous; it is staged into LDS with 16-byte loads, all
// issued before any use, and every product then runs from LDS.
template <int DK, int DV, typename IT, typename OT>
__global__ __launch_bounds__(NTHR) void scan_kernel(const IT* __restrict__ v,
                                                   const float* __restrict__ S0,
                                                   OT* __restrict__ o,
                                                   float* __restrict__ S_final, int L, int nc,
                                                   const float* __restrict__ ws) {
  constexpr int LDK = ScanSmem<DK>::LDK, LDC = ScanSmem<DK>::LDC;
  constexpr int RSTRIDE = NTHR / NT;  // rows between a thread's outputs
  constexpr int MR = C / RSTRIDE;    // chunk rows per thread
  constexpr int MS = DK / RSTRIDE;   // state rows per thread
  static_assert(MR >= 1 && MS >= 1 && MR * RSTRIDE == C && MS * RSTRIDE == DK, "thread map");
  constexpr int NF4 = (int)(chunk_floats(DK) / 4);
  static_assert(chunk_floats(DK) % 4 == 0 && (C * C) % 4 == 0 && (C * DK) % 4 == 0 && DK % 4 == 0,
                "16-byte pieces never straddle two tiles");
  extern __shared__ float smem[];
  float* Ts = smem;              // T
  float* Ps = Ts + C * LDC;      // P
  float* Kd = Ps + C * LDC;      // K o e^g
  float* Qd = Kd + C * LDK;      // Q o e^g
  float* Ku = Qd + C * LDK;      // K o e^{g_C - g}
  float* Ss = Ku + C * LDK;      // state columns j0 .. j0 + 15
  float* Rs = Ss + DK * NT;
  float* Ds = Rs + C * NT;
  float* gam = Ds + C * NT;      // e^{g_C}

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
    const float4* src = reinterpret_cast<const float4*>(ws + ((size_t)bh * nc + c) * chunk_floats(DK));
#pragma unroll 8
    for (int e4 = threadIdx.x; e4 < NF4; e4 += NTHR) {
      const float4 x = src[e4];
      int f = 4 * e4;
      float* dst;
      if (f < C * C) {
        dst = Ts + (f / C) * LDC + f % C;
      } else if ((f -= C * C) < C * C) {
        dst = Ps + (f / C) * LDC + f % C;
      } else if ((f -= C * C) < 3 * C * DK) {
        const int t = f / (C * DK), g = f % (C * DK);
        dst = Kd + t * C * LDK + (g / DK) * LDK + g % DK;
      } else {
        dst = gam + (f - 3 * C * DK);
      }
      dst[0] = x.x;
      dst[1] = x.y;
      dst[2] = x.z;
      dst[3] = x.w;
    }
    float vr[MR];
    for (int m = 0; m < MR; ++m) {
      const int r = rb + m * RSTRIDE;
      vr[m] = r < valid ? to_f32(v[(tok0 + r) * DV + j0 + j]) : 0.f;
    }
    __syncthreads();

    // R = V - (K o e^g) S into LDS; (Q o e^g) S kept in registers.
    float oi[MR];
    for (int m = 0; m < MR; ++m) {
      const int r = rb + m * RSTRIDE;
      float ks = 0.f, qs = 0.f;
#pragma unroll 8
      for (int d = 0; d < DK; ++d) {
        const float sd = Ss[d * NT + j];
        ks += Kd[r * LDK + d] * sd;
        qs += Qd[r * LDK + d] * sd;
      }
      Rs[r * NT + j] = vr[m] - ks;
      oi[m] = qs;
    }
    __syncthreads();

    // Delta = T R.
    for (int m = 0; m < MR; ++m) {
      const int r = rb + m * RSTRIDE;
      float acc = 0.f;
#pragma unroll 8
      for (int i = 0; i <= r; ++i) acc += Ts[r * LDC + i] * Rs[i * NT + j];
      Ds[r * NT + j] = acc;
    }
    __syncthreads();

    // O = (Q o e^g) S + P Delta, and S' = diag(e^{g_C}) S + (K o e^{g_C - g})^T Delta
    // (both read Delta; the state was last read before the previous barrier).
    for (int m = 0; m < MR; ++m) {
      const int r = rb + m * RSTRIDE;
      if (r < valid) {
        float acc = oi[m];
#pragma unroll 8
        for (int i = 0; i <= r; ++i) acc += Ps[r * LDC + i] * Ds[i * NT + j];
        o[(tok0 + r) * DV + j0 + j] = from_f32<OT>(acc);
      }
    }
    for (int m = 0; m < MS; ++m) {
      const int d = rb + m * RSTRIDE;
      float acc = gam[d] * Ss[d * NT + j];
#pragma unroll 8
      for (int r = 0; r < C; ++r) acc += Ku[r * LDK + d] * Ds[r * NT + j];
      Ss[d * NT + j] = acc;
    }
    __syncthreads();  // the next chunk overwrites every tile
  }

  if (S_final) {
    for (int m = 0; m < MS; ++m) {
      const int d = rb + m * RSTRIDE;
      S_final[sbase + (size_t)d * DV + j0 + j] = Ss[d * NT + j];
    }
  }
}

template <int DK, int DV, typename IT, typename OT>
hipError_t launch_t(const ChunkArgs& a) {
  const int nc = cdiv(a.L, C);
  const int bh = a.B * a.H;
  float* ws = static_cast<float*>(a.workspace);
  if constexpr (sizeof(IT) == 2) {  // bf16 q, k: the prep's products on the matrix cores
    if (nc > 0) {
      prof_mark(kSlotChunkPrep, false, a.stream);
      const hipError_t e =
          launch_prep_mfma(DK, a.q, a.k, a.alpha, a.beta, a.L, nc, bh, ws, a.stream);
      prof_mark(kSlotChunkPrep, true, a.stream);
      if (e != hipSuccess) return e;
    }
  } else if (nc > 0) {
    constexpr size_t sm = PrepSmem<DK>::bytes;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prep_kernel<DK, IT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    if (e != hipSuccess) return e;
    prof_mark(kSlotChunkPrep, false, a.stream);
    hipLaunchKernelGGL((prep_kernel<DK, IT>), dim3(nc, bh), dim3(NTHR), sm, a.stream,
                       static_cast<const IT*>(a.q), static_cast<const IT*>(a.k), a.alpha, a.beta,
                       a.L, ws);
    e = hipGetLastError();
    prof_mark(kSlotChunkPrep, true, a.stream);
    if (e != hipSuccess) return e;
  }
  if constexpr (sizeof(IT) == 2) {  // bf16 v: the scan runs on the matrix cores
    prof_mark(kSlotChunkScan, false, a.stream);
    const hipError_t e = launch_scan_mfma(DK, DV, a.out_dtype, a.v, a.S0, a.o, a.S_final, a.L, nc,
                                          bh, ws, a.stream);
    prof_mark(kSlotChunkScan, true, a.stream);
    return e;
  } else {
    constexpr size_t sm2 = ScanSmem<DK>::bytes;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_kernel<DK, DV, IT, OT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm2);
    if (e != hipSuccess) return e;
    prof_mark(kSlotChunkScan, false, a.stream);
    hipLaunchKernelGGL((scan_kernel<DK, DV, IT, OT>), dim3(DV / NT, bh), dim3(NTHR), sm2,
                       a.stream, static_cast<const IT*>(a.v), a.S0, static_cast<OT*>(a.o),
                       a.S_final, a.L, nc, ws);
    e = hipGetLastError();
    prof_mark(kSlotChunkScan, true, a.stream);
    return e;
  }
}

template <int DK, int DV>
hipError_t launch_types(const ChunkArgs& a) {
  if (a.in_dtype == 0 && a.out_dtype == 0) return launch_t<DK, DV, float, float>(a);
  if (a.in_dtype == 0 && a.out_dtype == 1) return launch_t<DK, DV, float, bf16>(a);
  if (a.in_dtype == 1 && a.out_dtype == 0) return launch_t<DK, DV, bf16, float>(a);
  return launch_t<DK, DV, bf16, bf16>(a);
}

}  // namespace kda

size_t kda_workspace_bytes(int B, int H, int L, int d_k) {
  return (size_t)B * H * cdiv(L, kda::C) * kda::chunk_floats(d_k) * sizeof(float);
}

hipError_t launch_kda_chunk_fwd(const ChunkArgs& a) {
  if (a.d_k == 64 && a.d_v == 64) return kda::launch_types<64, 64>(a);
  if (a.d_k == 64 && a.d_v == 128) return kda::launch_types<64, 128>(a);
  if (a.d_k == 128 && a.d_v == 64) return kda::launch_types<128, 64>(a);
  return kda::launch_types<128, 128>(a);
}

}  // namespace dn
