// dn_features.h -- the DeltaNet layer's feature maps as device functions,
// shared by the streaming feature kernel (dn_features.hip) and the decode
// step that applies them in-kernel (dn_decode.hip).
//
// The layer forward of the page "GPT-2 から Kimi K3 まで、AI モデルの進化を解説",
// section "DeltaNet (Fast weight programmers)", feeds the delta rule with
//     q = normalise(silu(q)),  k = normalise(silu(k))   (L2, along the head),
//     beta = sigmoid(logit),
// where normalise(x) = x / max(||x||_2, 1e-12) (PyTorch's F.normalize).
//
// Precision: silu and sigmoid take the hardware exp2 and reciprocal
// (v_exp_f32 on x log2(e), v_rcp_f32), a few fp32 ulps for |x| up to ~20
// (the error grows as |x| 2^-24 through the rounded exponent); the per-row
// norm uses the correctly rounded sqrt and division, once per row.  Squares
// are summed in fp32, so a row with elements beyond ~1e19 overflows.
#pragma once

#include <hip/hip_runtime.h>

#include "dn_common.h"

namespace dn {

constexpr float kNormalizeEps = 1e-12f;

__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

// silu(x) = x sigmoid(x); for x << 0, e^{-x} overflows to inf and the
// result is -0.
__device__ __forceinline__ float fast_silu(float x) { return x * fast_sigmoid(x); }

// 1 / max(sqrt(sum of squares), eps): the factor each element of the row is
// multiplied by.
__device__ __forceinline__ float inv_row_norm(float sumsq) {
  return 1.f / fmaxf(sqrtf(sumsq), kNormalizeEps);
}

// Row pieces of 16 bytes (8 bf16 or 4 fp32), used by the streaming feature
// kernel and by the WY-prep kernel that applies the maps as it loads k and q
// (the same arithmetic in the same order, so both give the same bits).
namespace feat {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void unpack(const uint4& w, float (&f)[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack(const uint4& w, float (&f)[4]) {
  f[0] = __uint_as_float(w.x);
  f[1] = __uint_as_float(w.y);
  f[2] = __uint_as_float(w.z);
  f[3] = __uint_as_float(w.w);
}
__device__ __forceinline__ uint4 pack(const float (&f)[8]) {
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    u[i] = f32x2_to_bf16x2_bits(f[2 * i], f[2 * i + 1]);
  return make_uint4(u[0], u[1], u[2], u[3]);
}
__device__ __forceinline__ uint4 pack(const float (&f)[4]) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                    __float_as_uint(f[3]));
}

// One row piece: silu, the row's norm across its LPR lanes, the scaled
// result packed back to the storage type.
template <int LPR, int V>
__device__ __forceinline__ uint4 map_piece(const uint4& in) {
  float f[V];
  unpack(in, f);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    f[i] = fast_silu(f[i]);
    ss += f[i] * f[i];
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float r = inv_row_norm(ss);
#pragma unroll
  for (int i = 0; i < V; ++i) f[i] *= r;
  return pack(f);
}

}  // namespace feat

}  // namespace dn
