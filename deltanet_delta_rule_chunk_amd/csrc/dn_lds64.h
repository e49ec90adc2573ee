// dn_lds64.h -- LDS operand helpers of the 64-row-chunk matrix-core kernels
// (the backward's kernels and the per-dimension-decay scan): fragment reads
// of bf16 arrays, split stores of accumulator tiles, and swizzled transposed
// copies whose contraction runs over the 64 chunk rows.
//
// A fragment read `frag(a, P, r0, kb)` gives lane l the 8 contraction slots
// kb + 8 (l / 16) ... of row r0 + l % 16 of a bf16 array with row pitch P:
// the A layout of the 16 x 16 x 32 MFMA and, for an array stored
// [column][contraction], its B layout.
#pragma once

#include "dn_mfma.h"

namespace dn {
namespace lds64 {

constexpr int C = 64;      // chunk rows
constexpr int PC = C + 8;  // pitch (bf16) of arrays whose contraction runs over chunk rows

__device__ __forceinline__ bf16x8 frag(const uint16_t* a, int P, int r0, int kb) {
  const int l = threadIdx.x & 63;
  return as_bf16x8(*reinterpret_cast<const uint4*>(a + (r0 + (l & 15)) * P + kb + 8 * (l >> 4)));
}

// A D tile (lane: column l % 16, rows r0 + 4 (l / 16) + e) split into hi and
// lo and stored transposed, hi[column * P + row].
__device__ __forceinline__ void put_split_t(uint16_t* hi, uint16_t* lo, int P, int r0, f32x4 v) {
  const int l = threadIdx.x & 63;
  uint2 h, o;
  split4(v, h, o);
  const int off = (l & 15) * P + r0 + 4 * (l >> 4);
  *reinterpret_cast<uint2*>(hi + off) = h;
  *reinterpret_cast<uint2*>(lo + off) = o;
}

// Transposed copies ([column][chunk row], 8 chunks of 8 rows per line) have
// their 16-byte chunks XOR-swizzled by a function of the line, so that
// deposits with consecutive lanes along the source rows hit distinct banks:
//   lines from a C x DK tile: chunk ^ ((line >> 3) & 7)   (SH = 3)
//   lines from a C x C block: chunk ^ ((line >> 2) & 7)   (SH = 2)
template <int SH>
__device__ __forceinline__ int tpos(int line, int row) {
  return line * PC + ((((row >> 3) ^ (line >> SH)) & 7) << 3) + (row & 7);
}

// frag() for a swizzled transposed copy.
template <int SH>
__device__ __forceinline__ bf16x8 fragT(const uint16_t* a, int r0, int kb) {
  const int l = threadIdx.x & 63, line = r0 + (l & 15);
  const int ch = (((kb >> 3) + (l >> 4)) ^ (line >> SH)) & 7;
  return as_bf16x8(*reinterpret_cast<const uint4*>(a + line * PC + (ch << 3)));
}

// Stores a D tile (lane: column l % 16, rows 4 (l / 16) + e) into a
// row-major fp32 matrix (dst = the tile's top-left element, row pitch ld)
// straight from the accumulators: four 4-byte stores per lane, each covering
// 64 contiguous bytes of four rows.  (Going through an LDS tile to store 16
// bytes per lane instead put an LDS round trip on the caller's path and was
// measured slower.)  Rows at or past `rows` are not stored.
__device__ __forceinline__ void store_tile16(f32x4 v, float* dst, size_t ld, int rows = 16) {
  const int l = threadIdx.x & 63, n = l & 15, g = l >> 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * g + e;
    if (row < rows) dst[row * ld + n] = v[e];
  }
}

// 8 fp32 values -> split bf16x8 pair.
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
  uint2 h0, l0, h1, l1;
  split4(make_float4(x[0], x[1], x[2], x[3]), h0, l0);
  split4(make_float4(x[4], x[5], x[6], x[7]), h1, l1);
  hi = as_bf16x8(h0, h1);
  lo = as_bf16x8(l0, l1);
}

}  // namespace lds64
}  // namespace dn
