// dn_common.h -- device helpers shared by the library's gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dn {

// bf16 is carried as its 16-bit pattern.  fp32 -> bf16 rounds to nearest,
// ties to even (gfx950's v_cvt_pk_bf16_f32, which converts two values per
// instruction; NaN stays NaN).
struct bf16 {
  uint16_t bits;
};
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) {
  return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// (a, b) -> bf16 bits of a in the low half, of b in the high half.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
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
