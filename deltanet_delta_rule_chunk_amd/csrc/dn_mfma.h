// dn_mfma.h -- gfx950 matrix-core helpers: the 16x16x32 bf16 MFMA and the
// split of fp32 values into bf16 (hi, lo) pairs.
//
// v_mfma_f32_16x16x32_bf16 operand layout (wave64, lane l, g = l / 16,
// i = l % 16):
//   A (16 x 32): lane holds row i, contraction slots 8g .. 8g+7
//   B (32 x 16): lane holds column i, contraction slots 8g .. 8g+7
//   D (16 x 16, fp32): lane holds column i, rows 4g .. 4g+3
// Only the pairing of A's and B's slots matters for the sum, so a product
// may map its contraction index to the slots in any order, provided both
// operands use the same map.  Two maps are used here:
//   "row8":  slot (g, e) <-> k = 8g + e            (16-byte operand reads)
//   "d4":    slot (g, e) <-> k = 4g + e (e < 4),  16 + 4g + (e - 4) (e >= 4)
//            which is exactly what two stacked D tiles of an earlier product
//            hold per lane, so a result can feed the next product from
//            registers.
//
// Split precision: an fp32 value x is carried as hi = bf16(x) and
// lo = bf16(x - hi), both rounded to nearest even; the product of two split
// values is taken as hi*hi + hi*lo + lo*hi (the lo*lo term is below 2^-16
// relative).  A bf16-exact operand (the stored q, k) times a split one needs
// two passes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 h = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, h);
}

// Splits (a, b) into packed hi and lo bf16 pairs.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(a, b);
  const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xffff0000u);
  lo = pack_bf16(a - ha, b - hb);
}

// Splits four fp32 values into 4 hi and 4 lo bf16 (8 bytes each).
__device__ __forceinline__ void split4(f32x4 v, uint2& hi, uint2& lo) {
  split2(v[0], v[1], hi.x, lo.x);
  split2(v[2], v[3], hi.y, lo.y);
}

__device__ __forceinline__ void split4(float4 v, uint2& hi, uint2& lo) {
  split2(v.x, v.y, hi.x, lo.x);
  split2(v.z, v.w, hi.y, lo.y);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ bf16x8 as_bf16x8(uint2 a, uint2 b) {
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// acc += (a_hi + a_lo)(b_hi + b_lo) without the lo*lo term.
__device__ __forceinline__ f32x4 mfma_split3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl,
                                             f32x4 acc) {
  acc = mfma16(ah, bh, acc);
  acc = mfma16(ah, bl, acc);
  acc = mfma16(al, bh, acc);
  return acc;
}

// acc += a (b_hi + b_lo), a exact in bf16.
__device__ __forceinline__ f32x4 mfma_split2(bf16x8 a, bf16x8 bh, bf16x8 bl, f32x4 acc) {
  acc = mfma16(a, bh, acc);
  acc = mfma16(a, bl, acc);
  return acc;
}

}  // namespace dn
