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

}  // namespace dn
