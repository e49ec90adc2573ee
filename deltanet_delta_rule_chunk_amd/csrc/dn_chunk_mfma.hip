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
// Kernels:
//   prep_kernel  one 4-wave workgroup per (chunk, head), all chunks in
//                parallel.  Gram blocks K K^T on bf16 MFMA (bf16 products are
//                exact, sums in fp32), the unit-lower inverse (I + A)^{-1} by
//                recursive doubling [[X1,0],[A21,X2]] -> X21 = -X2 A21 X1 with
//                split-bf16 MFMA products, then T = X diag(beta) written to
//                the workspace as ready-made MFMA operand fragments (hi and lo
//                bf16 planes, lower-triangular blocks only).
//   scan_kernel  one 8-wave workgroup per (head, 16-column slice of d_v):
//                walks the chunks in order; the state slice (d_k x 16, fp32)
//                lives in MFMA accumulator registers.  Columns of S evolve
//                independently, so the d_v slices are independent scans.
//                Per chunk: R = V - K S, Delta = T R, O = Q S + P Delta with
//                P = tril(Q K^T) formed on the fly, S += K^T Delta.
// Every fp32 operand of a product (S, R, Delta, T, P, and inside the
// inverse) is carried as a (hi, lo) bf16 pair; q, k (bf16 inputs) are exact.
// A ragged last chunk reads zero rows of k, q, v and beta = 0, which makes
// the padded rows and columns of T zero: exact no-ops.

#include "dn_common.h"
#include "dn_launch.h"
#include "dn_mfma.h"

namespace dn {
namespace mf {

// Layout of T's fragments per chunk: row tile t (16 rows) owns the k-blocks
// kb = 0 .. t/2 (32 columns each) of the lower triangle; block (t, kb) is
// 2 planes (hi, lo) x 64 lanes x 16 bytes, lane (g, i) holding
// T[16t + i][32kb + 8g .. 8g + 7].
template <int C>
struct Frag {
  static constexpr int NT = C / 16;
  __host__ __device__ static constexpr int base(int t) {
    return (t & 1) ? (t / 2 + 1) * (t / 2 + 1) : (t / 2) * (t / 2 + 1);
  }
  static constexpr int NBLK = base(NT);
  static constexpr size_t chunk_u4 = (size_t)NBLK * 2 * 64;  // uint4 per chunk
};

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

// ---------------------------------------------------------------------------
// scan_kernel
// ---------------------------------------------------------------------------

template <int C, int DK>
struct ScanCfg {
  static constexpr int NW = (C == 128 || DK == 128) ? 8 : 4;  // waves per workgroup
  static constexpr int NTHR = NW * 64;
  static constexpr int KLD = DK + 8;  // bf16 pitch of K and Q tiles
  static constexpr int TLD = C + 8;   // bf16 pitch of the transposed K tile
  static constexpr size_t bytes =
      (2 * (size_t)C * KLD + (size_t)DK * TLD + 2 * (size_t)DK * 16 + 4 * (size_t)C * 16) *
      sizeof(uint16_t);
};

// Offset (in bf16 elements, within one hi or lo plane) of element (x, j) of a
// [rows x 16] operand stored in row8 fragment order: [x/32][(x%32)/8][j][x%8].
__device__ __forceinline__ int frag_off(int x, int j) {
  return ((x >> 5) * 4 + ((x & 31) >> 3)) * 128 + j * 8 + (x & 7);
}

// Issues the global loads of chunk cc into registers: this thread's share of
// the k and q tiles (RPT rows x 8 columns), and for a wave with a row tile rt
// its v values (D layout) and T fragments.  Rows past L read as zero.
template <int C, int DK, int DV, int RPT, int NKB>
__device__ __forceinline__ void load_chunk(const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ k,
                                           const uint16_t* __restrict__ v,
                                           const uint4* __restrict__ Tfrag, int bh, int L, int nc,
                                           int cc, int sr0, int sd0, int rt, int g, int i16,
                                           int lane, int j0, uint4 (&kst)[RPT], uint4 (&qst)[RPT],
                                           uint32_t (&vst)[4], uint4 (&tst)[2 * NKB]) {
  const int t0 = cc * C, valid = min(C, L - t0);
  const size_t tok0 = (size_t)bh * L + t0;
  // Loads always read an in-bounds row (clamped to the last valid one) and
  // select zero afterwards, so the register arrays are written without
  // branches.
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = sr0 + i;
    const size_t rr = tok0 + min(r, valid - 1);
    kst[i] = *reinterpret_cast<const uint4*>(k + rr * DK + sd0);
    qst[i] = *reinterpret_cast<const uint4*>(q + rr * DK + sd0);
  }
  if (rt >= 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * rt + 4 * g + r;
      vst[r] = v[(tok0 + min(row, valid - 1)) * DV + j0 + i16];
    }
    const uint4* tb =
        Tfrag + ((size_t)bh * nc + cc) * Frag<C>::chunk_u4 + (size_t)Frag<C>::base(rt) * 2 * 64;
    // Blocks past the tile's last one (kb > rt/2) are never used; they
    // re-read block 0 so every array slot is written unconditionally.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int blk = (kb <= rt / 2) ? kb : 0;
      tst[2 * kb] = tb[(2 * blk) * 64 + lane];
      tst[2 * kb + 1] = tb[(2 * blk + 1) * 64 + lane];
    }
  }
}

template <int C, int DK, int DV, typename OT>
__global__ __launch_bounds__((ScanCfg<C, DK>::NTHR)) void scan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ S0, OT* __restrict__ o,
    float* __restrict__ S_final, int L, int nc, int BH, const uint4* __restrict__ Tfrag) {
  using CF = ScanCfg<C, DK>;
  constexpr int NW = CF::NW, NTHR = CF::NTHR, KLD = CF::KLD, TLD = CF::TLD;
  constexpr int NROW = C / 16, NDT = DK / 16, NCT = DV / 16;
  constexpr int NKB = NROW / 2;          // 32-wide k-blocks over the chunk
  constexpr int RPT = C * DK / (NTHR * 8);  // staged rows per thread
  constexpr int TPR = DK / 8;               // threads per staged row
  static_assert(RPT == 2 || RPT == 4, "staging shape");

  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem_raw);
  uint16_t* Qs = Ks + C * KLD;
  uint16_t* Kt = Qs + C * KLD;
  uint16_t* Sb = Kt + DK * TLD;  // hi plane, lo plane at + DK * 16
  uint16_t* Rb = Sb + 2 * DK * 16;
  uint16_t* Db = Rb + 2 * C * 16;

  // Workgroup -> (head, column slice).  Workgroups are handed to the 8 XCDs
  // round-robin by flat id, so all slices of a head share flat id mod 8 and
  // run on one XCD, whose L2 then serves their common k, q and T reads.
  const int flat = blockIdx.x;
  const int xcd = flat & 7, slot = flat >> 3;
  const int ct = slot % NCT, bh = (slot / NCT) * 8 + xcd;
  if (bh >= BH) return;
  const int j0 = ct * 16;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, i16 = lane & 15;
  // Row tile of this wave; waves w and w + 4 share a SIMD, so pair tiles
  // (t, 7 - t) to balance the triangular products.
  int rt = -1;
  if (NROW == 8 && NW == 8) rt = (w < 4) ? w : 11 - w;
  else if (w < NROW) rt = w;
  const bool has_row = rt >= 0;
  const bool has_dt = w < NDT;
  const int dt = w;

  const size_t sbase = (size_t)bh * DK * DV;
  f32x4 s = zero4();
  if (has_dt && S0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = S0[sbase + (size_t)(16 * dt + 4 * g + r) * DV + j0 + i16];
  }

  const int sd0 = 8 * (tid % TPR), sr0 = RPT * (tid / TPR);
  uint4 kst[RPT], qst[RPT], tst[2 * NKB], tcur[2 * NKB];
  uint32_t vst[4], vcur[4];

#define DN_LOAD_CHUNK(cc)                                                                   \
  load_chunk<C, DK, DV, RPT, NKB>(q, k, v, Tfrag, bh, L, nc, (cc), sr0, sd0, rt, g, i16, lane, \
                                  j0, kst, qst, vst, tst)
  if (nc > 0) DN_LOAD_CHUNK(0);

  for (int cc = 0; cc < nc; ++cc) {
    const int t0 = cc * C, valid = min(C, L - t0);
    const size_t tok0 = (size_t)bh * L + t0;

    // (1) Staged k, q -> LDS (k both ways); state slice -> split operand.
    // Rows past L were loaded from a clamped (valid) row; they are zeroed
    // here, at first use, so the loads above stay in flight until now.
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const uint32_t m = (sr0 + i) < valid ? 0xffffffffu : 0u;
      kst[i] = make_uint4(kst[i].x & m, kst[i].y & m, kst[i].z & m, kst[i].w & m);
      qst[i] = make_uint4(qst[i].x & m, qst[i].y & m, qst[i].z & m, qst[i].w & m);
      *reinterpret_cast<uint4*>(Ks + (sr0 + i) * KLD + sd0) = kst[i];
      *reinterpret_cast<uint4*>(Qs + (sr0 + i) * KLD + sd0) = qst[i];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t h[RPT];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const uint32_t word = (e < 2) ? kst[i].x : (e < 4) ? kst[i].y : (e < 6) ? kst[i].z : kst[i].w;
        h[i] = (e & 1) ? (word >> 16) : (word & 0xffffu);
      }
      uint16_t* dst = Kt + (sd0 + e) * TLD + sr0;
      if constexpr (RPT == 4) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      } else {
        *reinterpret_cast<uint32_t*>(dst) = h[0] | (h[1] << 16);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) vcur[i] = (16 * rt + 4 * g + i) < valid ? vst[i] : 0u;
#pragma unroll
    for (int i = 0; i < 2 * NKB; ++i) tcur[i] = tst[i];
    if (has_dt) {
      uint2 hi, lo;
      split4(s, hi, lo);
      const int off = frag_off(16 * dt + 4 * g, i16);
      *reinterpret_cast<uint2*>(Sb + off) = hi;
      *reinterpret_cast<uint2*>(Sb + DK * 16 + off) = lo;
    }
    __syncthreads();

    // (2) Prefetch the next chunk; R = V - K S, O = Q S, P^T blocks.
    if (cc + 1 < nc) DN_LOAD_CHUNK(cc + 1);
    f32x4 oacc = zero4();
    uint4 pah[NKB], pal[NKB];
    if (has_row) {
      f32x4 racc = zero4();
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const bf16x8 Sh = as_bf16x8(lds16(Sb + (kb * 4 + g) * 128 + i16 * 8));
        const bf16x8 Sl = as_bf16x8(lds16(Sb + DK * 16 + (kb * 4 + g) * 128 + i16 * 8));
        const bf16x8 Ka = as_bf16x8(lds16(Ks + (16 * rt + i16) * KLD + 32 * kb + 8 * g));
        const bf16x8 Qa = as_bf16x8(lds16(Qs + (16 * rt + i16) * KLD + 32 * kb + 8 * g));
        racc = mfma_split2(Ka, Sh, Sl, racc);
        oacc = mfma_split2(Qa, Sh, Sl, oacc);
      }
      f32x4 R;
#pragma unroll
      for (int r = 0; r < 4; ++r) R[r] = bf16_bits_to_f32(vcur[r]) - racc[r];
      uint2 hi, lo;
      split4(R, hi, lo);
      const int off = frag_off(16 * rt + 4 * g, i16);
      *reinterpret_cast<uint2*>(Rb + off) = hi;
      *reinterpret_cast<uint2*>(Rb + C * 16 + off) = lo;

      // P^T[c'][c] = K[c'] . Q[c] for the wave's rows c; D tiles hold
      // P[c = 16 rt + i16][c' = 16 b + 4g + r], the d4 slot map of an A operand.
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        f32x4 p0 = zero4(), p1 = zero4();
        if (kb <= rt / 2) {
          const bool second = (2 * kb + 1) <= rt;
#pragma unroll
          for (int d = 0; d < DK / 32; ++d) {
            const bf16x8 Qb = as_bf16x8(lds16(Qs + (16 * rt + i16) * KLD + 32 * d + 8 * g));
            const bf16x8 K0 = as_bf16x8(lds16(Ks + (32 * kb + i16) * KLD + 32 * d + 8 * g));
            p0 = mfma16(K0, Qb, p0);
            if (second) {
              const bf16x8 K1 = as_bf16x8(lds16(Ks + (32 * kb + 16 + i16) * KLD + 32 * d + 8 * g));
              p1 = mfma16(K1, Qb, p1);
            }
          }
          if (2 * kb == rt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) if (4 * g + r > i16) p0[r] = 0.f;
          }
          if (2 * kb + 1 == rt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) if (4 * g + r > i16) p1[r] = 0.f;
          }
        }
        uint2 h0, l0, h1, l1;
        split4(p0, h0, l0);
        split4(p1, h1, l1);
        pah[kb] = make_uint4(h0.x, h0.y, h1.x, h1.y);
        pal[kb] = make_uint4(l0.x, l0.y, l1.x, l1.y);
      }
    }
    __syncthreads();

    // (3) Delta = T R.
    if (has_row) {
      f32x4 dacc = zero4();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if (kb <= rt / 2) {
          const bf16x8 Rh = as_bf16x8(lds16(Rb + (kb * 4 + g) * 128 + i16 * 8));
          const bf16x8 Rl = as_bf16x8(lds16(Rb + C * 16 + (kb * 4 + g) * 128 + i16 * 8));
          dacc = mfma_split3(as_bf16x8(tcur[2 * kb]), as_bf16x8(tcur[2 * kb + 1]), Rh, Rl, dacc);
        }
      }
      uint2 hi, lo;
      split4(dacc, hi, lo);
      const int off = frag_off(16 * rt + 4 * g, i16);
      *reinterpret_cast<uint2*>(Db + off) = hi;
      *reinterpret_cast<uint2*>(Db + C * 16 + off) = lo;
    }
    __syncthreads();

    // (4) S += K^T Delta;  O += P Delta.
    if (has_dt) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 Ka = as_bf16x8(lds16(Kt + (16 * dt + i16) * TLD + 32 * kb + 8 * g));
        const bf16x8 Dh = as_bf16x8(lds16(Db + (kb * 4 + g) * 128 + i16 * 8));
        const bf16x8 Dl = as_bf16x8(lds16(Db + C * 16 + (kb * 4 + g) * 128 + i16 * 8));
        s = mfma_split2(Ka, Dh, Dl, s);
      }
    }
    if (has_row) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if (kb <= rt / 2) {
          const int o0 = (kb * 4 + (g >> 1)) * 128 + i16 * 8 + 4 * (g & 1);
          const int o1 = o0 + 2 * 128;
          const uint2 dh0 = lds8(Db + o0), dh1 = lds8(Db + o1);
          const uint2 dl0 = lds8(Db + C * 16 + o0), dl1 = lds8(Db + C * 16 + o1);
          oacc = mfma_split3(as_bf16x8(pah[kb]), as_bf16x8(pal[kb]), as_bf16x8(dh0, dh1),
                             as_bf16x8(dl0, dl1), oacc);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rt + 4 * g + r;
        if (row < valid) o[(tok0 + row) * DV + j0 + i16] = from_f32<OT>(oacc[r]);
      }
    }
    __syncthreads();
  }

#undef DN_LOAD_CHUNK
  if (S_final && has_dt) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S_final[sbase + (size_t)(16 * dt + 4 * g + r) * DV + j0 + i16] = s[r];
  }
}

template <int C, int DK, int DV, typename OT>
hipError_t launch_t(const ChunkArgs& a) {
  const int nc = cdiv(a.L, C);
  const int BH = a.B * a.H;
  uint4* Tfrag = static_cast<uint4*>(a.workspace);
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  hipError_t e;
  if (nc > 0) {
    constexpr size_t sm = PrepSmem<C, DK>::bytes;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prep_kernel<C, DK>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    if (e != hipSuccess) return e;
    prof_mark(kSlotChunkPrep, false, a.stream);
    hipLaunchKernelGGL((prep_kernel<C, DK>), dim3(nc, BH), dim3(256), sm, a.stream, k, a.beta,
                       a.L, nc, Tfrag);
    e = hipGetLastError();
    prof_mark(kSlotChunkPrep, true, a.stream);
    if (e != hipSuccess) return e;
  }
  using CF = ScanCfg<C, DK>;
  constexpr size_t sm2 = CF::bytes;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_kernel<C, DK, DV, OT>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm2);
  if (e != hipSuccess) return e;
  const int groups = cdiv(BH, 8) * 8 * (DV / 16);
  prof_mark(kSlotChunkScan, false, a.stream);
  hipLaunchKernelGGL((scan_kernel<C, DK, DV, OT>), dim3(groups), dim3(CF::NTHR), sm2, a.stream,
                     q, k, v, a.S0, static_cast<OT*>(a.o), a.S_final, a.L, nc, BH, Tfrag);
  e = hipGetLastError();
  prof_mark(kSlotChunkScan, true, a.stream);
  return e;
}

template <int C, int DK, int DV>
hipError_t launch_o(const ChunkArgs& a) {
  return a.out_dtype == 0 ? launch_t<C, DK, DV, float>(a) : launch_t<C, DK, DV, bf16>(a);
}

template <int C>
hipError_t launch_c(const ChunkArgs& a) {
  if (a.d_k == 64 && a.d_v == 64) return launch_o<C, 64, 64>(a);
  if (a.d_k == 64 && a.d_v == 128) return launch_o<C, 64, 128>(a);
  if (a.d_k == 128 && a.d_v == 64) return launch_o<C, 128, 64>(a);
  return launch_o<C, 128, 128>(a);
}

}  // namespace mf

size_t chunk_workspace_bytes_mfma(int B, int H, int L, int C) {
  const size_t nc = (size_t)cdiv(L, C);
  const size_t per = C == 64 ? mf::Frag<64>::chunk_u4 : mf::Frag<128>::chunk_u4;
  return (size_t)B * H * nc * per * sizeof(uint4);
}

hipError_t launch_chunk_fwd_mfma(const ChunkArgs& a) {
  return a.C == 64 ? mf::launch_c<64>(a) : mf::launch_c<128>(a);
}

}  // namespace dn
