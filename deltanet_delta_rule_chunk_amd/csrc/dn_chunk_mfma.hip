// dn_chunk_mfma.hip -- chunkwise-parallel delta-rule forward for bf16 inputs
// on gfx950 matrix cores: the WY-prep kernel and the launch sequence (the
// state scan that consumes T is in dn_scan_mfma.hip).
//
// The chunked form (page "GPT-2 から Kimi K3 まで、AI モデルの進化を解説",
// section "DeltaNet (Parallelizing linear transformers with delta rule)":
// each chunk's outputs follow from the previous chunk's final state and the
// chunk's own q, k, v, through generalised-Householder transitions; the
// printed reparameterisation is cut off, so it is written out here from the
// recurrence).  For a chunk with rows K, beta:
//     A = tril(diag(beta) K K^T, -1),    T = (I + A)^{-1} diag(beta),
// so that (I + A) T = diag(beta), T is lower triangular and diag(T) = beta.
//
// prep_kernel: one 4-wave workgroup per (chunk, head), all chunks in
// parallel, ~68 KB of LDS so two workgroups share a CU.  With 16 x 16 tiles
// (NT = C / 16 tile rows):
//   1. k rows -> LDS (swizzled, dn_ktile.h).
//   2. Gram tiles on bf16 MFMA (bf16 products are exact, sums fp32); the
//      off-diagonal tiles of A are kept as split-bf16 MFMA operands, the
//      diagonal tiles' strictly lower parts N_i as fp32.
//   3. The unit-lower 16 x 16 inverses Linv_i = (I + N_i)^{-1} by fp32
//      forward substitution, one lane per column.
//   4. Column tiles of T by block forward substitution: tile column j of
//      (I + A) T = diag(beta) is independent of the other tile columns:
//          T_jj = Linv_j diag(beta_j),
//          T_ij = Linv_i R_ij,  R_ij = -sum_{j <= k < i} A_ik T_kj   (i > j).
//      Each wave owns whole tile columns and keeps them in registers.  T_ij
//      comes out of one MFMA in column layout (the B operand of the next
//      row's products) and its transpose R_ij^T Linv_i^T from another in row
//      layout (the stored A operand) -- both from the same split registers.
// Every fp32 operand of a product is carried as a (hi, lo) bf16 pair, the
// product taken as hi*hi + hi*lo + lo*hi.  A ragged last chunk reads zero
// rows of k and beta = 0, which makes the padded rows and columns of T zero.

#include "dn_common.h"
#include "dn_ktile.h"
#include "dn_launch.h"
#include "dn_mfma.h"
#include "dn_tfrag.h"

namespace dn {

hipError_t launch_scan_mfma(const ChunkArgs& a, const uint4* Tfrag);

namespace prep {

template <int C, int DK>
struct Cfg {
  static constexpr int NT = C / 16;                    // 16-row tiles
  static constexpr int NKB = DK / 32;                  // 32-wide blocks of d_k
  static constexpr int NOFF = NT * (NT - 1) / 2;       // off-diagonal lower tiles
  static constexpr int SPT = C * DK / (8 * 256);       // staged 16-byte k pieces per thread
  // LDS, in bytes.  Region 0 holds the k tile, later the two fp32 layouts of
  // the diagonal inverses.
  static constexpr int R0 = C * DK * 2 > NT * 2048 ? C * DK * 2 : NT * 2048;
  static constexpr int OFF_A = R0;                     // NOFF tiles x 2 planes x 512 B
  static constexpr int OFF_N = OFF_A + NOFF * 1024;    // NT tiles x 1 KB fp32
  static constexpr int OFF_BETA = OFF_N + NT * 1024;   // C floats
  static constexpr size_t bytes = (size_t)OFF_BETA + C * 4;
  static_assert(SPT >= 1, "shape");
};

// Lower tile (i, k), i > k, of A: index in the off-diagonal list.
__device__ __forceinline__ int tidx(int i, int k) { return i * (i - 1) / 2 + k; }

__device__ __forceinline__ bf16x8 lds16(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(p));
}

template <int C, int DK>
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ k,
                                                   const float* __restrict__ beta, int L,
                                                   int nc, uint4* __restrict__ Tfrag) {
  using CF = Cfg<C, DK>;
  constexpr int NT = CF::NT, NKB = CF::NKB;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint16_t* const Ks = reinterpret_cast<uint16_t*>(smem_raw);
  float* const Lrow = reinterpret_cast<float*>(smem_raw);             // after step 2
  float* const Lcol = reinterpret_cast<float*>(smem_raw) + NT * 256;  // after step 2
  uint2* const Atl = reinterpret_cast<uint2*>(smem_raw + CF::OFF_A);
  float* const Nd = reinterpret_cast<float*>(smem_raw + CF::OFF_N);
  float* const bs = reinterpret_cast<float*>(smem_raw + CF::OFF_BETA);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, i16 = lane & 15;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int t0 = c * C, valid = min(C, L - t0);
  const size_t tok0 = (size_t)bh * L + t0;

  // ---- 1. k tile and beta -> LDS --------------------------------------------
  {
    uint4 kv[CF::SPT];
#pragma unroll
    for (int i = 0; i < CF::SPT; ++i) {
      const int e = i * 256 + tid, row = e / (DK / 8), ch = e % (DK / 8);
      kv[i] = *reinterpret_cast<const uint4*>(k + (tok0 + min(row, valid - 1)) * DK + ch * 8);
    }
    if (tid < C) bs[tid] = tid < valid ? beta[tok0 + tid] : 0.f;
#pragma unroll
    for (int i = 0; i < CF::SPT; ++i) {
      const int e = i * 256 + tid, row = e / (DK / 8), ch = e % (DK / 8);
      const uint32_t m = row < valid ? 0xffffffffu : 0u;
      *reinterpret_cast<uint4*>(Ks + koff<DK>(row, ch)) =
          make_uint4(kv[i].x & m, kv[i].y & m, kv[i].z & m, kv[i].w & m);
    }
  }
  __syncthreads();

  // ---- 2. Gram tiles -----------------------------------------------------------
  // Tile (i, kk), kk <= i, computed as K_kk K_i^T so that lane (i16, g)
  // register r holds G[16 i + i16][16 kk + 4 g + r]: A_{i,kk} in row layout.
  constexpr int NTT = NT * (NT + 1) / 2;
  for (int p = w; p < NTT; p += 4) {
    int i = 0;
    while ((i + 1) * (i + 2) / 2 <= p) ++i;
    const int kk = p - i * (i + 1) / 2;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const bf16x8 Ak = lds16(Ks + koff<DK>(16 * kk + i16, 4 * kb + g));
      const bf16x8 Bi = lds16(Ks + koff<DK>(16 * i + i16, 4 * kb + g));
      acc = mfma16(Ak, Bi, acc);
    }
    const float b = bs[16 * i + i16];
    if (i > kk) {
      uint2 hi, lo;
      split4(acc * b, hi, lo);
      Atl[tidx(i, kk) * 128 + lane] = hi;
      Atl[tidx(i, kk) * 128 + 64 + lane] = lo;
    } else {
      // Strictly lower part of the diagonal tile, stored column-major:
      // Nd[i][col][row] = N_i[row][col].
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = 4 * g + r;
        Nd[i * 256 + col * 16 + i16] = col < i16 ? acc[r] * b : 0.f;
      }
    }
  }
  __syncthreads();

  // ---- 3. Linv_b = (I + N_b)^{-1}, one lane per (block b, column cc) ----------
  // Column-oriented substitution: once x_kk is final, every later row
  // subtracts N[row][kk] x_kk.  Column kk of N_b is one broadcast read.
  if (tid < 16 * NT) {
    const int b = tid >> 4, cc = tid & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = r == cc ? 1.f : 0.f;
#pragma unroll
    for (int kk = 0; kk < 15; ++kk) {
      float ncol[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 v = *reinterpret_cast<const float4*>(Nd + b * 256 + kk * 16 + 4 * q4);
        ncol[4 * q4] = v.x; ncol[4 * q4 + 1] = v.y; ncol[4 * q4 + 2] = v.z; ncol[4 * q4 + 3] = v.w;
      }
#pragma unroll
      for (int r = kk + 1; r < 16; ++r) x[r] -= ncol[r] * x[kk];
    }
    // Row layout: lane (row, g) of a consumer holds Linv[row][4 g .. 4 g + 3].
#pragma unroll
    for (int r = 0; r < 16; ++r) Lrow[b * 256 + (16 * (cc >> 2) + r) * 4 + (cc & 3)] = x[r];
    // Column layout: lane (col, g) holds Linv[4 g .. 4 g + 3][col].
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<float4*>(Lcol + b * 256 + (16 * q4 + cc) * 4) =
          make_float4(x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]);
  }
  __syncthreads();

  // ---- 4. tile columns of T ------------------------------------------------------
  uint4* const out = Tfrag + ((size_t)bh * nc + c) * Frag<C>::chunk_u4;
  // 8-byte half (j & 1) of block (i, j / 2), both planes, this lane.
  auto tstore = [&](int i, int j, uint2 hi, uint2 lo) {
    uint2* blk = reinterpret_cast<uint2*>(out + (size_t)(Frag<C>::base(i) + j / 2) * 128);
    blk[2 * lane + (j & 1)] = hi;
    blk[128 + 2 * lane + (j & 1)] = lo;
  };
  constexpr int NCOLW = NT > 4 ? 2 : 1;  // tile columns per wave
#pragma unroll
  for (int cw = 0; cw < NCOLW; ++cw) {
    const int j = cw == 0 ? w : NT - 1 - w;
    // Column layout of T_kj (lane (i16, g) holds T_kj[4 g + r][i16]), split.
    uint2 th[NT], tl[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) { th[t] = make_uint2(0u, 0u); tl[t] = th[t]; }
    {
      const f32x4 lc = *reinterpret_cast<const f32x4*>(Lcol + j * 256 + lane * 4);
      const float bcol = bs[16 * j + i16];
      uint2 hi, lo;
      split4(lc * bcol, hi, lo);
#pragma unroll
      for (int t = 0; t < NT; ++t) if (t == j) { th[t] = hi; tl[t] = lo; }
      const f32x4 lr = *reinterpret_cast<const f32x4*>(Lrow + j * 256 + lane * 4);
      const float4 brow = *reinterpret_cast<const float4*>(bs + 16 * j + 4 * g);
      f32x4 trow;
      trow[0] = lr[0] * brow.x; trow[1] = lr[1] * brow.y;
      trow[2] = lr[2] * brow.z; trow[3] = lr[3] * brow.w;
      split4(trow, hi, lo);
      tstore(j, j, hi, lo);
      if (j & 1) tstore(j - 1, j, make_uint2(0u, 0u), make_uint2(0u, 0u));
    }
#pragma unroll
    for (int i = 1; i < NT; ++i) {
      if (i <= j) continue;
      // R_ij = -sum_k A_ik T_kj over tile pairs (2p, 2p + 1); T_kj = 0 for
      // k < j and A_ik is only taken for k < i.
      f32x4 a0 = zero4(), a1 = zero4(), a2 = zero4();
#pragma unroll
      for (int p = 0; p < NT / 2; ++p) {
        if (2 * p > i - 1 || 2 * p + 1 < j) continue;
        const uint2 z = make_uint2(0u, 0u);
        const uint2 ah0 = Atl[tidx(i, 2 * p) * 128 + lane], al0 = Atl[tidx(i, 2 * p) * 128 + 64 + lane];
        const bool two = 2 * p + 1 < i;
        const uint2 ah1 = two ? Atl[tidx(i, 2 * p + 1) * 128 + lane] : z;
        const uint2 al1 = two ? Atl[tidx(i, 2 * p + 1) * 128 + 64 + lane] : z;
        const bf16x8 Ah = as_bf16x8(ah0, ah1), Al = as_bf16x8(al0, al1);
        const bf16x8 Bh = as_bf16x8(th[2 * p], th[2 * p + 1]), Bl = as_bf16x8(tl[2 * p], tl[2 * p + 1]);
        a0 = mfma16(Ah, Bh, a0);
        a1 = mfma16(Ah, Bl, a1);
        a2 = mfma16(Al, Bh, a2);
      }
      const f32x4 R = -(a0 + a1 + a2);
      uint2 rh, rl;
      split4(R, rh, rl);
      const f32x4 lr = *reinterpret_cast<const f32x4*>(Lrow + i * 256 + lane * 4);
      uint2 lh, ll;
      split4(lr, lh, ll);
      const uint2 z = make_uint2(0u, 0u);
      const bf16x8 Lh = as_bf16x8(lh, z), Ll = as_bf16x8(ll, z);
      const bf16x8 Rh = as_bf16x8(rh, z), Rl = as_bf16x8(rl, z);
      // T_ij = Linv_i R_ij (column layout, kept for the next rows).
      f32x4 tc = mfma16(Lh, Rh, zero4());
      tc = mfma16(Lh, Rl, tc);
      tc = mfma16(Ll, Rh, tc);
      split4(tc, th[i], tl[i]);
      // T_ij^T = R_ij^T Linv_i^T (row layout, stored).
      f32x4 tr = mfma16(Rh, Lh, zero4());
      tr = mfma16(Rh, Ll, tr);
      tr = mfma16(Rl, Lh, tr);
      uint2 hi, lo;
      split4(tr, hi, lo);
      tstore(i, j, hi, lo);
    }
  }
}

template <int C, int DK>
hipError_t launch_c(const ChunkArgs& a) {
  const int nc = cdiv(a.L, C);
  const int BH = a.B * a.H;
  uint4* Tfrag = static_cast<uint4*>(a.workspace);
  if (nc > 0) {
    constexpr size_t sm = Cfg<C, DK>::bytes;
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

}  // namespace prep

size_t chunk_workspace_bytes_mfma(int B, int H, int L, int C) {
  const size_t nc = (size_t)cdiv(L, C);
  const size_t per = C == 64 ? Frag<64>::chunk_u4 : Frag<128>::chunk_u4;
  return (size_t)B * H * nc * per * sizeof(uint4);
}

hipError_t launch_chunk_fwd_mfma(const ChunkArgs& a) {
  if (a.C == 64) return a.d_k == 64 ? prep::launch_c<64, 64>(a) : prep::launch_c<64, 128>(a);
  return a.d_k == 64 ? prep::launch_c<128, 64>(a) : prep::launch_c<128, 128>(a);
}

}  // namespace dn
