// dn_chunk_mfma.hip -- chunkwise-parallel delta-rule forward for bf16 inputs
// on gfx950 matrix cores.
//
// The chunked form (page "GPT-2 から Kimi K3 まで、AI モデルの進化を解説",
// section "DeltaNet (Parallelizing linear transformers with delta rule)":
// each chunk's outputs follow from the previous chunk's final state and the
// chunk's own q, k, v, through generalised-Householder transitions; the
// printed reparameterisation is cut off, so it is written out here from the
// recurrence).  For a chunk with rows K, Q, V, beta and entering state S:
//     A     = tril(diag(beta) K K^T, -1)
//     T     = (I + A)^{-1} diag(beta)        (lower triangular; diag(T) = beta)
//     Delta = T (V - K S)                    (all of the chunk's deltas at once)
//     O     = Q S + tril(Q K^T) Delta        (masked attention inside the chunk,
//                                             diagonal included, plus the read
//                                             of the state between chunks)
//     S'    = S + K^T Delta
//
// This file holds the WY-prep kernel and the launch sequence; the state scan
// that consumes T is in dn_scan_mfma.hip.
//   prep_kernel  one 4-wave workgroup per (chunk, head), all chunks in
//                parallel.  Gram blocks K K^T on bf16 MFMA (bf16 products are
//                exact, sums in fp32), the unit-lower inverse (I + A)^{-1} by
//                recursive doubling [[X1,0],[A21,X2]] -> X21 = -X2 A21 X1 with
//                split-bf16 MFMA products, then T = X diag(beta) written to
//                the workspace as ready-made MFMA operand fragments (hi and lo
//                bf16 planes, lower-triangular blocks only; dn_tfrag.h).
// Every fp32 operand of a product inside the inverse is carried as a
// (hi, lo) bf16 pair; k (bf16 input) is exact.  A ragged last chunk reads
// zero rows of k and beta = 0, which makes the padded rows and columns of T
// zero: exact no-ops.

#include "dn_common.h"
#include "dn_launch.h"
#include "dn_mfma.h"
#include "dn_tfrag.h"

namespace dn {

hipError_t launch_scan_mfma(const ChunkArgs& a, const uint4* Tfrag);

namespace mf {

__device__ __forceinline__ uint4 lds16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ uint2 lds8(const uint16_t* p) {
  return *reinterpret_cast<const uint2*>(p);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// ---------------------------------------------------------------------------
// prep_kernel
// ---------------------------------------------------------------------------

template <int C, int DK>
struct PrepSmem {
  static constexpr int MLD = C + 4;   // fp32 pitch of M and Mt
  static constexpr int KLD = DK + 8;  // bf16 pitch of the K tile
  static constexpr size_t bytes = (2 * (size_t)C * MLD + C) * sizeof(float);
  static_assert((size_t)C * KLD * 2 <= (size_t)C * MLD * 4, "K tile must fit in Mt");
};

// One doubling level: for every pair of S x S diagonal blocks (X1 above,
// X2 below, A21 the block of A between them) X21 = -X2 (A21 X1).  Wave w
// owns 16-column tile w of the C/32 column tiles of all X21 blocks of the
// level (every level has exactly C/32 of them).
template <int C, int S>
__device__ __forceinline__ void invert_level(float* M, float* Mt, int w, int g, int i16) {
  constexpr int MLD = C + 4;
  constexpr int RT = S / 16;            // 16-row tiles of Y and X21
  constexpr int KB = (S + 31) / 32;     // 32-wide k-blocks over S
  constexpr int CTP = S / 16;           // column tiles per pair
  const bool active = w < C / 32;
  f32x4 x21[RT];
  int r0 = 0, ct = 0;
  if (active) {
    const int p = w / CTP;
    ct = w % CTP;
    r0 = 2 * p * S;
    const bool slot_ok = (S >= 32) || (g < 2);  // S = 16: slots 16..31 are padding
    f32x4 y[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) y[rt] = zero4();
    // Y = A21 X1 (row8 slot map; X1 read as columns from the transposed copy).
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (kb < ct / 2) continue;  // X1[k][col] = 0 for k < col
      float4 b0 = make_float4(0.f, 0.f, 0.f, 0.f), b1 = b0;
      if (slot_ok) {
        const float* pb = Mt + (r0 + 16 * ct + i16) * MLD + r0 + 32 * kb + 8 * g;
        b0 = *reinterpret_cast<const float4*>(pb);
        b1 = *reinterpret_cast<const float4*>(pb + 4);
      }
      uint2 bh0, bl0, bh1, bl1;
      split4(b0, bh0, bl0);
      split4(b1, bh1, bl1);
      const bf16x8 Bh = as_bf16x8(bh0, bh1), Bl = as_bf16x8(bl0, bl1);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
        if (slot_ok) {
          const float* pa = M + (r0 + S + 16 * rt + i16) * MLD + r0 + 32 * kb + 8 * g;
          a0 = *reinterpret_cast<const float4*>(pa);
          a1 = *reinterpret_cast<const float4*>(pa + 4);
        }
        uint2 ah0, al0, ah1, al1;
        split4(a0, ah0, al0);
        split4(a1, ah1, al1);
        y[rt] = mfma_split3(as_bf16x8(ah0, ah1), as_bf16x8(al0, al1), Bh, Bl, y[rt]);
      }
    }
    // X21 = -X2 Y (d4 slot map: Y's D tiles feed the B operand from registers).
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (kb > rt / 2) continue;  // X2[row][k] = 0 for k > row
        const f32x4 ylo = y[2 * kb];
        const f32x4 yhi = (2 * kb + 1 < RT) ? y[(2 * kb + 1) % RT] : zero4();
        uint2 bh0, bl0, bh1, bl1;
        split4(ylo, bh0, bl0);
        split4(yhi, bh1, bl1);
        const float* pa = M + (r0 + S + 16 * rt + i16) * MLD + r0 + S + 32 * kb + 4 * g;
        const float4 a0 = *reinterpret_cast<const float4*>(pa);
        const float4 a1 = (2 * kb + 1 < RT) ? *reinterpret_cast<const float4*>(pa + 16)
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
        uint2 ah0, al0, ah1, al1;
        split4(a0, ah0, al0);
        split4(a1, ah1, al1);
        acc = mfma_split3(as_bf16x8(ah0, ah1), as_bf16x8(al0, al1), as_bf16x8(bh0, bh1),
                          as_bf16x8(bl0, bl1), acc);
      }
      x21[rt] = -acc;
    }
  }
  __syncthreads();  // every wave is done reading A21, X1, X2
  if (active) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int x = r0 + S + 16 * rt + 4 * g, y = r0 + 16 * ct + i16;
#pragma unroll
      for (int r = 0; r < 4; ++r) M[(x + r) * MLD + y] = x21[rt][r];
      *reinterpret_cast<float4*>(Mt + y * MLD + x) =
          make_float4(x21[rt][0], x21[rt][1], x21[rt][2], x21[rt][3]);
    }
  }
  __syncthreads();
}

template <int C, int DK>
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ k,
                                                   const float* __restrict__ beta, int L,
                                                   int nc, uint4* __restrict__ Tfrag) {
  using SM = PrepSmem<C, DK>;
  constexpr int MLD = SM::MLD, KLD = SM::KLD;
  constexpr int NB = C / 16;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float* M = reinterpret_cast<float*>(smem_raw);
  float* Mt = M + C * MLD;
  uint16_t* Ks = reinterpret_cast<uint16_t*>(Mt);  // aliases Mt until the Gram blocks are done
  float* bs = Mt + C * MLD;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, i16 = lane & 15;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int t0 = c * C, valid = min(C, L - t0);
  const size_t tok0 = (size_t)bh * L + t0;

  constexpr int V8 = DK / 8;
  for (int e = tid; e < C * V8; e += 256) {
    const int r = e / V8, cv = e % V8;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (r < valid) val = *reinterpret_cast<const uint4*>(k + (tok0 + r) * DK + cv * 8);
    *reinterpret_cast<uint4*>(Ks + r * KLD + cv * 8) = val;
  }
  for (int r = tid; r < C; r += 256) bs[r] = r < valid ? beta[tok0 + r] : 0.f;
  for (int e = tid; e < C * MLD / 4; e += 256)
    reinterpret_cast<float4*>(M)[e] = make_float4(0.f, 0.f, 0.f, 0.f);
  __syncthreads();

  // Gram blocks (a, b), a >= b, and A = tril(diag(beta) G, -1) into M.
  constexpr int NBP = NB * (NB + 1) / 2;
  for (int p = w; p < NBP; p += 4) {
    int a = 0;
    while ((a + 1) * (a + 2) / 2 <= p) ++a;
    const int b = p - a * (a + 1) / 2;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
      const bf16x8 A = as_bf16x8(lds16(Ks + (16 * a + i16) * KLD + 32 * kb + 8 * g));
      const bf16x8 B = as_bf16x8(lds16(Ks + (16 * b + i16) * KLD + 32 * kb + 8 * g));
      acc = mfma16(A, B, acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int x = 16 * a + 4 * g + r, y = 16 * b + i16;
      M[x * MLD + y] = (y < x) ? bs[x] * acc[r] : 0.f;
    }
  }
  __syncthreads();
  for (int e = tid; e < C * MLD / 4; e += 256)
    reinterpret_cast<float4*>(Mt)[e] = make_float4(0.f, 0.f, 0.f, 0.f);
  __syncthreads();

  // Diagonal 16 x 16 blocks of X = (I + A)^{-1}: column y of a unit-lower
  // block depends only on earlier rows of the same column.
  float xcol[16];
  if (tid < C) {
    const int b = tid / 16, jj = tid % 16, y = 16 * b + jj;
#pragma unroll
    for (int xi = 0; xi < 16; ++xi) {
      float val = 0.f;
      if (xi == jj) {
        val = 1.f;
      } else if (xi > jj) {
        float acc = 0.f;
#pragma unroll
        for (int zi = 0; zi < xi; ++zi)
          if (zi >= jj) acc += M[(16 * b + xi) * MLD + 16 * b + zi] * xcol[zi];
        val = -acc;
      }
      xcol[xi] = val;
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<float4*>(Mt + y * MLD + 16 * b + 4 * q4) =
          make_float4(xcol[4 * q4], xcol[4 * q4 + 1], xcol[4 * q4 + 2], xcol[4 * q4 + 3]);
  }
  __syncthreads();
  if (tid < C) {
    const int b = tid / 16, y = tid;
#pragma unroll
    for (int xi = 0; xi < 16; ++xi) M[(16 * b + xi) * MLD + y] = xcol[xi];
  }
  __syncthreads();

  invert_level<C, 16>(M, Mt, w, g, i16);
  invert_level<C, 32>(M, Mt, w, g, i16);
  if constexpr (C == 128) invert_level<C, 64>(M, Mt, w, g, i16);

  // T = X diag(beta) as hi/lo fragments.
  constexpr int NBLK = Frag<C>::NBLK;
  uint4* out = Tfrag + ((size_t)bh * nc + c) * Frag<C>::chunk_u4;
  for (int blk = w; blk < NBLK; blk += 4) {
    int t = 0;
    while (t + 1 < NB && Frag<C>::base(t + 1) <= blk) ++t;
    const int kb = blk - Frag<C>::base(t);
    const int x = 16 * t + i16, y0 = 32 * kb + 8 * g;
    float vals[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int y = y0 + e;
      vals[e] = (y <= x) ? M[x * MLD + y] * bs[y] : 0.f;
    }
    uint4 hi, lo;
    split2(vals[0], vals[1], hi.x, lo.x);
    split2(vals[2], vals[3], hi.y, lo.y);
    split2(vals[4], vals[5], hi.z, lo.z);
    split2(vals[6], vals[7], hi.w, lo.w);
    out[(blk * 2 + 0) * 64 + lane] = hi;
    out[(blk * 2 + 1) * 64 + lane] = lo;
  }
}

template <int C, int DK>
hipError_t launch_c(const ChunkArgs& a) {
  const int nc = cdiv(a.L, C);
  const int BH = a.B * a.H;
  uint4* Tfrag = static_cast<uint4*>(a.workspace);
  if (nc > 0) {
    constexpr size_t sm = PrepSmem<C, DK>::bytes;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prep_kernel<C, DK>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    if (e != hipSuccess) return e;
    prof_mark(kSlotChunkPrep, false, a.stream);
    hipLaunchKernelGGL((prep_kernel<C, DK>), dim3(nc, BH), dim3(256), sm, a.stream,
                       static_cast<const uint16_t*>(a.k), a.beta, a.L, nc, Tfrag);
    e = hipGetLastError();
    prof_mark(kSlotChunkPrep, true, a.stream);
    if (e != hipSuccess) return e;
  }
  return launch_scan_mfma(a, Tfrag);
}

}  // namespace mf

size_t chunk_workspace_bytes_mfma(int B, int H, int L, int C) {
  const size_t nc = (size_t)cdiv(L, C);
  const size_t per = C == 64 ? Frag<64>::chunk_u4 : Frag<128>::chunk_u4;
  return (size_t)B * H * nc * per * sizeof(uint4);
}

hipError_t launch_chunk_fwd_mfma(const ChunkArgs& a) {
  if (a.C == 64) return a.d_k == 64 ? mf::launch_c<64, 64>(a) : mf::launch_c<64, 128>(a);
  return a.d_k == 64 ? mf::launch_c<128, 64>(a) : mf::launch_c<128, 128>(a);
}

}  // namespace dn
