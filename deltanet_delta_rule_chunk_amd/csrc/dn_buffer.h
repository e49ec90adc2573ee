// dn_buffer.h -- raw buffer loads through descriptors held in scalar
// registers, for kernels that walk a sequence chunk by chunk: the chunk's
// base address goes into the descriptor (made once per chunk, uniform), each
// lane keeps a fixed byte offset, so a load spends no vector instructions on
// its address; and a read at or past the descriptor's byte count returns
// zero, which turns rows past the end of a ragged last chunk into zeros.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dn {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Descriptor over `bytes` bytes from `base` (raw access, stride 0).  Both
// arguments must be the same in every lane; they are read from the first
// lane so that the descriptor lives in scalar registers.  (readfirstlane
// returns a signed int: each half of the address goes through uint32_t so
// that widening it never sign-extends into the other half.)
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
// Loads of 16, 8 and 4 bytes at byte offset voff + soff (soff uniform).
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint2 bload8(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

}  // namespace dn
