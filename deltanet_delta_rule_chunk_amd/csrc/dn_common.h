// dn_common.h -- device helpers shared by the library's gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dn {

// bf16 is carried as its 16-bit pattern; conversions are written out here so
// the rounding rule is explicit (round to nearest, ties to even).
struct bf16 {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) {
  return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) {
  return bf16{f32_to_bf16_bits(x)};
}

// log(alpha) of a decay alpha in [0, 1], floored at log(FLT_MIN) so that a
// zero decay (a full wipe) becomes a factor e^{-87.3} ~ 1e-38 and every
// difference of summed log-decays stays finite.
constexpr float kLogDecayFloor = -87.33654f;
__device__ __forceinline__ float log_decay(float alpha) {
  return alpha > 0.f ? fmaxf(logf(alpha), kLogDecayFloor) : kLogDecayFloor;
}

// Ceil-divide for launch geometry.
__host__ __device__ constexpr inline int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace dn
