// dn_features.hip -- the layer's feature maps as one streaming kernel:
//     q_hat = normalise(silu(q_raw)),  k_hat = normalise(silu(k_raw)),
//     beta  = sigmoid(beta_logit)
// (page "GPT-2 から Kimi K3 まで、AI モデルの進化を解説", section "DeltaNet (Fast
// weight programmers)"; the maps are in dn_features.h).  q_hat and k_hat are
// stored in the input dtype (bf16: rounded to nearest, ties to even), beta
// in fp32.
//
// The kernel reads every input byte once and writes every output byte once,
// so it is bound by HBM bandwidth: per row of d_k it moves 4 d_k (bf16) or
// 8 d_k (fp32) bytes of q and k in each direction plus 8 bytes of beta.  Its
// arithmetic (an exp and a reciprocal per element) is close to that bound on
// the vector ALUs when packed fp32 is off, so each element takes the
// hardware exp2 and reciprocal and only the per-row norm takes the exact
// sqrt and division.
//
// Layout: a row is d_k contiguous elements; LPR = d_k / (elements per 16
// bytes) adjacent lanes hold one row, 16 bytes each, so a wave's loads are
// whole, adjacent rows.  The row's sum of squares is reduced across its LPR
// lanes with xor shuffles (every lane ends with the same sum: the butterfly
// adds the same two partial sums in both lanes of a pair).  A 256-thread
// workgroup takes U = 4 passes of 256 / LPR rows, all loads issued first.
// Loads and stores are non-temporal: every byte is touched once, and keeping
// the streams out of the caches measured ~4% faster at 2 GiB per launch
// (5.8 TB/s, against 5.2 TB/s for the runtime's device-to-device copy of the
// same bytes).
// Each lane writes only what it read itself, after reading it, so the maps
// may run in place (an output buffer equal to its input); the pointers are
// therefore not declared restrict.
// The fused chunked forward runs this kernel into its workspace and then the
// chunk kernels on the mapped operands.

#include "dn_common.h"
#include "dn_features.h"
#include "dn_launch.h"

namespace dn {
namespace feat {

constexpr int NT = 256;
constexpr int U = 4;

template <typename T>
struct Pack {
  static constexpr int N = 16 / sizeof(T);  // elements per 16 bytes
};

template <int DK, typename T>
__global__ __launch_bounds__(NT) void feature_kernel(const T* q_raw, const T* k_raw,
                                                     const float* beta_logit, T* q_hat, T* k_hat,
                                                     float* beta, long long N) {
  constexpr int V = Pack<T>::N;
  constexpr int LPR = DK / V;     // lanes per row
  constexpr int RPP = NT / LPR;   // rows per pass
  constexpr int RPB = RPP * U;    // rows per workgroup
  static_assert(LPR * V == DK && LPR <= 64 && 64 % LPR == 0, "row shape");
  static_assert(RPB <= NT, "one beta per thread");

  const long long row0 = (long long)blockIdx.x * RPB;
  const int lane_in_row = threadIdx.x % LPR, rsub = threadIdx.x / LPR;
  uint4 xq[U], xk[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const long long row = row0 + u * RPP + rsub;
    xq[u] = xk[u] = make_uint4(0, 0, 0, 0);
    if (row < N) {
      const size_t off = (size_t)row * DK + lane_in_row * V;
      const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q_raw + off));
      const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_raw + off));
      xq[u] = make_uint4(a.x, a.y, a.z, a.w);
      xk[u] = make_uint4(b.x, b.y, b.z, b.w);
    }
  }
  float bl = 0.f;
  const long long brow = row0 + threadIdx.x;
  if (threadIdx.x < RPB && brow < N) bl = beta_logit[brow];

#pragma unroll
  for (int u = 0; u < U; ++u) {
    // Rows past N hold zeros: their lanes still join the shuffles (all
    // lanes of a wave must) and then store nothing.
    const long long row = row0 + u * RPP + rsub;
    const uint4 oq = map_piece<LPR, V>(xq[u]);
    const uint4 ok = map_piece<LPR, V>(xk[u]);
    if (row < N) {
      const size_t off = (size_t)row * DK + lane_in_row * V;
      __builtin_nontemporal_store(u32x4{oq.x, oq.y, oq.z, oq.w}, reinterpret_cast<u32x4*>(q_hat + off));
      __builtin_nontemporal_store(u32x4{ok.x, ok.y, ok.z, ok.w}, reinterpret_cast<u32x4*>(k_hat + off));
    }
  }
  if (threadIdx.x < RPB && brow < N) beta[brow] = fast_sigmoid(bl);
}

template <int DK, typename T>
constexpr int rows_per_block() {
  return NT / (DK / Pack<T>::N) * U;
}

template <int DK, typename T>
static hipError_t launch_t(const FeatureArgs& a) {
  constexpr int RPB = rows_per_block<DK, T>();
  const long long blocks = (a.rows + RPB - 1) / RPB;
  if (blocks == 0) return hipSuccess;
  prof_mark(kSlotFeatures, false, a.stream);
  hipLaunchKernelGGL((feature_kernel<DK, T>), dim3((unsigned)blocks), dim3(NT), 0, a.stream,
                     static_cast<const T*>(a.q_raw), static_cast<const T*>(a.k_raw),
                     a.beta_logit, static_cast<T*>(a.q_hat), static_cast<T*>(a.k_hat), a.beta,
                     a.rows);
  hipError_t e = hipGetLastError();
  prof_mark(kSlotFeatures, true, a.stream);
  return e;
}

}  // namespace feat

long long feature_max_rows(int d_k, int dtype) {
  const int rpb = dtype == 1 ? (d_k == 64 ? feat::rows_per_block<64, bf16>()
                                          : feat::rows_per_block<128, bf16>())
                             : (d_k == 64 ? feat::rows_per_block<64, float>()
                                          : feat::rows_per_block<128, float>());
  return (long long)rpb * 0x7fffffffLL;
}

hipError_t launch_features(const FeatureArgs& a) {
  if (a.dtype == 1)
    return a.d_k == 64 ? feat::launch_t<64, bf16>(a) : feat::launch_t<128, bf16>(a);
  return a.d_k == 64 ? feat::launch_t<64, float>(a) : feat::launch_t<128, float>(a);
}

}  // namespace dn
