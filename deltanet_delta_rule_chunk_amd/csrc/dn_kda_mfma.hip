// dn_kda_mfma.hip -- the per-dimension-decay (KDA) scan on the gfx950 matrix
// cores, for bf16 v.
//
// Same products as the vector-ALU scan in dn_kda.hip, chunk by chunk from
// the prep kernel's workspace (T, P, K o e^g, Q o e^g, K o e^{g_C - g},
// e^{g_C}):
//     R  = V - (K o e^g) S,        Delta = T R,
//     O  = (Q o e^g) S + P Delta,  S' = diag(e^{g_C}) S + (K o e^{g_C - g})^T Delta.
// Every operand is an fp32 value, which the prep stores as a split (hi, lo)
// bf16 pair (two planes per matrix block, in the bytes of the fp32 block), so
// each product is taken as three 16 x 16 x 32 bf16 MFMAs (dn_mfma.h),
// accumulated in fp32.
//
// One 4-wave workgroup per (head, 16 columns of d_v); the slice of the state
// lives in MFMA accumulators (wave w holds row tiles w d_k / 64 ...).  Wave w
// owns chunk rows 16 w .. 16 w + 15 of R, Delta and O, so the row operands of
// those products (rows of K o e^g, Q o e^g, T and P) are private to it: each
// wave loads them from the workspace straight into fragment registers, a
// chunk ahead.  Only K o e^{g_C - g}, which the state update contracts over
// chunk rows, goes through LDS (transposed, split), together with the split
// state and the R and Delta columns that pass between the waves.  Four
// barriers per chunk: deposit, R (and (Q o e^g) S), Delta, O and S'.

#include "dn_common.h"
#include "dn_inv64.h"
#include "dn_kda.h"
#include "dn_lds64.h"
#include "dn_mfma.h"
#include "dn_valu_common.h"

namespace dn {
namespace kda {
namespace mf {

using lds64::frag;
using lds64::split8;
using lds64::fragT;
using lds64::PC;
using lds64::put_split_t;
using lds64::tpos;

constexpr int NTH = 256;   // 4 waves: one role of the scan
constexpr int SNTH = 512;  // the scan's workgroup: 4 chain + 4 output waves

// ---- prep ------------------------------------------------------------------
// The pair factors of A and P, e^{g_r - g_i} per dimension, are bounded
// (every exponent <= 0) but do not factor into matrix-core operands over a
// whole chunk.  Between 16-row blocks they do: for row r in block b > b' and
// row i in block b', with m = 16 b the first row of r's block,
//     e^{g_r - g_i} = e^{g_r - g_m} e^{g_m - g_i},
// and both exponents are <= 0 (g only decreases along the chunk).  So each
// of the six tiles below the block diagonal is a product of two bounded fp32
// operands, K o e^{g - g_m} (or Q o e^{g - g_m}) against K o e^{g_m - g},
// taken on the matrix cores with split operands (one wave per tile).  The
// four diagonal tiles keep the factor per (pair, dimension) on the vector
// ALUs (one thread per pair, on the other ten waves).  Then the blocked fp32
// inverse of I + A (dn_inv64.h).
constexpr int PNTHR = 1024;

// 8 consecutive values as split pairs, one 16-byte store per plane (i is a
// multiple of 8).
// (Non-temporal stores here measured the same time but 1.8 GB more HBM
// writes per long-context launch.)
__device__ __forceinline__ void put_split8(uint16_t* hi, int plane, int i, const float* x) {
  bf16x8 h, o;
  lds64::split8(x, h, o);
  *reinterpret_cast<bf16x8*>(hi + i) = h;
  *reinterpret_cast<bf16x8*>(hi + plane + i) = o;
}

// x as a split pair: hi[i] = bf16(x), hi[plane + i] = bf16(x - hi[i]).
__device__ __forceinline__ void put_split(uint16_t* hi, int plane, int i, float x) {
  const __bf16 h = static_cast<__bf16>(x);
  hi[i] = __builtin_bit_cast(uint16_t, h);
  hi[plane + i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x - static_cast<float>(h)));
}

template <int DK>
struct PrepLds {
  // K and Q stay in LDS as bf16 (exact: they are bf16 inputs); g, and later
  // X = (I + A)^{-1}, in fp32; A takes the bytes of K and Q once their last
  // reader is done.  About 72 KB at d_k = 128, so two workgroups share a CU
  // and one chunk's loads and stores overlap another's arithmetic.
  static constexpr int LDH = DK + 8;  // row pitch of the bf16 K and Q tiles (elements)
  static constexpr int LD = DK + 4;   // row pitch of the fp32 g tile and of X
  static constexpr int LDA = C + 1;   // row pitch of A
  static constexpr size_t kq_bytes = 2 * (size_t)C * LDH * 2;
  static_assert((size_t)C * LDA * 4 <= kq_bytes, "A over K and Q");
  static_assert(LD >= C, "X over g");
  static_assert(8 * DK <= inv64::SCRATCH_FLOATS, "prefix totals in the inverse's scratch");
  static constexpr size_t bytes = kq_bytes + ((size_t)C * LD + C + inv64::SCRATCH_FLOATS) * 4;
};

// 8 consecutive bf16 (16 bytes, aligned) as fp32.
__device__ __forceinline__ void bf8(const uint16_t* p, float* x) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t h[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(h[i] << 16);
    x[2 * i + 1] = __uint_as_float(h[i] & 0xffff0000u);
  }
}
// 4 consecutive bf16 (8 bytes, aligned) as fp32.
__device__ __forceinline__ float4 bf4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

// log2(alpha), floored at -120: a zero decay (a full wipe) becomes a factor
// 2^-120 ~ 7.5e-37.  The floor keeps a one-row factor 2^(g_{r+1} - g_r) a
// normal number even after the rounding of the summed log-decays (the
// diagonal pairs below multiply it by its reciprocal), and every difference
// of summed log-decays finite.  2^x runs on the hardware exponential.
__device__ __forceinline__ float log2_decay(float alpha) {
  return alpha > 0.f ? fmaxf(log2f(alpha), -120.f) : -120.f;
}
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DK>
__global__ __launch_bounds__(PNTHR) __attribute__((amdgpu_waves_per_eu(8))) void prep_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const float* __restrict__ alpha,
    const float* __restrict__ beta, int L, float* __restrict__ ws) {
  constexpr int LDH = PrepLds<DK>::LDH, LD = PrepLds<DK>::LD, LDA = PrepLds<DK>::LDA;
  constexpr int KS = DK / 32;
  constexpr size_t CF = chunk_floats(DK);
  extern __shared__ float smem_f[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem_f);  // K (bf16)
  uint16_t* Qs = Ks + C * LDH;                           // Q (bf16)
  float* As = smem_f;                                    // A, over K and Q after their last read
  // g, the cumulative log-decays, is held in base 2 (the sums of log2(alpha)),
  // so that every factor e^{g_a - g_b} is a single 2^x instruction.
  float* Gs = smem_f + PrepLds<DK>::kq_bytes / 4;        // g / ln 2, later X
  float* bs = Gs + C * LD;                               // beta
  float* scratch = bs + C;                               // the inverse's per-wave tiles

  const int c = blockIdx.x, bh = blockIdx.y, nc = gridDim.x;
  const int valid = min(C, L - c * C);
  const size_t tok0 = (size_t)bh * L + (size_t)c * C;
  // Each matrix block holds its split pair as two bf16 planes, hi then lo.
  float* blk = ws + ((size_t)bh * nc + c) * CF;
  uint16_t* Tc = reinterpret_cast<uint16_t*>(blk);
  uint16_t* Pc = Tc + 2 * C * C;
  uint16_t* Kd = Pc + 2 * C * C;   // K o e^g
  uint16_t* Qd = Kd + 2 * C * DK;  // Q o e^g
  uint16_t* Ku = Qd + 2 * C * DK;  // K o e^{g_C - g}
  float* gam = reinterpret_cast<float*>(Ku + 2 * C * DK);  // e^{g_C}
  const int t = threadIdx.x, l = t & 63, n = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // (wave-uniform: scalar)

  // Every global read of the chunk (q and k rows, 16 bytes per load, the
  // decays, beta) is issued before the first of them is waited on.
  constexpr int NKQ = (C * DK / 8 + PNTHR - 1) / PNTHR, NA = C * DK / (4 * PNTHR);
  static_assert(C * DK % (4 * PNTHR) == 0 && (C * DK / 8) % 64 == 0, "load shape");
  uint4 xk[NKQ], xq[NKQ];
  float4 av[NA];  // the decays, 4 consecutive dimensions per load
  {
    const uint4* kg = reinterpret_cast<const uint4*>(k + tok0 * DK);
    const uint4* qg = reinterpret_cast<const uint4*>(q + tok0 * DK);
#pragma unroll
    for (int it = 0; it < NKQ; ++it) {
      const int e8 = t + PNTHR * it, r = e8 / (DK / 8), c8 = e8 % (DK / 8);
      const int rc = min(r, valid - 1);
      if (e8 < C * DK / 8) {
        xk[it] = kg[rc * (DK / 8) + c8];
        xq[it] = qg[rc * (DK / 8) + c8];
      }
    }
#pragma unroll
    for (int it = 0; it < NA; ++it) {
      const int e = 4 * (t + PNTHR * it), r = e / DK, j = e % DK;
      av[it] = *reinterpret_cast<const float4*>(alpha + (tok0 + min(r, valid - 1)) * DK + j);
    }
  }
  const float bt = t < C && t < valid ? beta[tok0 + t] : 0.f;
#pragma unroll
  for (int it = 0; it < NKQ; ++it) {  // into the bf16 tiles as they are (rows past L: zeros)
    const int e8 = t + PNTHR * it, r = e8 / (DK / 8), c8 = e8 % (DK / 8);
    // (Masked lane by lane: a select between whole uint4 values was lowered
    // through private memory.)
    const uint32_t m = r < valid ? ~0u : 0u;
    const uint4 xkm = make_uint4(xk[it].x & m, xk[it].y & m, xk[it].z & m, xk[it].w & m);
    const uint4 xqm = make_uint4(xq[it].x & m, xq[it].y & m, xq[it].z & m, xq[it].w & m);
    if (e8 < C * DK / 8) {
      *reinterpret_cast<uint4*>(Ks + r * LDH + 8 * c8) = xkm;
      *reinterpret_cast<uint4*>(Qs + r * LDH + 8 * c8) = xqm;
    }
  }
  if (t < C) bs[t] = bt;
  // g: the log-decays of the whole tile at once (coalesced), then a prefix
  // sum down each dimension's column: 8 segments of 8 rows per column, each
  // summed in registers, then offset by the totals of the segments above it
  // (parked in the inverse's scratch, which is used only later).
#pragma unroll
  for (int it = 0; it < NA; ++it) {
    const int e = 4 * (t + PNTHR * it), r = e / DK, j = e % DK;
    const bool in = r < valid;
    *reinterpret_cast<float4*>(Gs + r * LD + j) =
        make_float4(in ? log2_decay(av[it].x) : 0.f, in ? log2_decay(av[it].y) : 0.f,
                    in ? log2_decay(av[it].z) : 0.f, in ? log2_decay(av[it].w) : 0.f);
  }
  __syncthreads();
  {
    static_assert(8 * DK <= PNTHR, "prefix layout");
    const int j = t % DK, seg = t / DK;
    float v[8];
    if (seg < 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = Gs[(8 * seg + i) * LD + j];
#pragma unroll
      for (int i = 1; i < 8; ++i) v[i] += v[i - 1];
      scratch[seg * DK + j] = v[7];
    }
    __syncthreads();
    if (seg < 8) {
      float off = 0.f;
      for (int s2 = 0; s2 < seg; ++s2) off += scratch[s2 * DK + j];
#pragma unroll
      for (int i = 0; i < 8; ++i) Gs[(8 * seg + i) * LD + j] = v[i] + off;
    }
  }
  __syncthreads();

  for (int e8 = t; e8 < C * DK / 8; e8 += PNTHR) {  // the decayed operands of the scan
    const int r = e8 / (DK / 8), j0 = 8 * (e8 % (DK / 8));
    float kv[8], qv[8], kd[8], qd[8], ku[8];
    bf8(Ks + r * LDH + j0, kv);
    bf8(Qs + r * LDH + j0, qv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float gv = Gs[r * LD + j0 + i], gC = Gs[(C - 1) * LD + j0 + i];
      kd[i] = kv[i] * exp2_raw(gv);
      qd[i] = qv[i] * exp2_raw(gv);
      ku[i] = kv[i] * exp2_raw(gC - gv);
    }
    put_split8(Kd, C * DK, 8 * e8, kd);
    put_split8(Qd, C * DK, 8 * e8, qd);
    put_split8(Ku, C * DK, 8 * e8, ku);
  }
  for (int j = t; j < DK; j += PNTHR) gam[j] = exp2_raw(Gs[(C - 1) * LD + j]);
  for (int e = t; e < C * C; e += PNTHR)  // P above the diagonal
    if (e % C > e / C) put_split(Pc, C * C, e, 0.f);

  // The entries of A below the diagonal, held in registers until K and Q
  // have no reader left, then written over them.
  f32x4 aa = zero4();
  float a = 0.f;
  int ar = 0, ai = 0;  // the vector-ALU pair's (row, column), a valid zero entry by default
  if (w < 6) {
    // Tile (br, bi) below the block diagonal; wave w takes tile w of
    // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2).
    const int br = w < 1 ? 1 : w < 3 ? 2 : 3;
    const int bi = w - (br * (br - 1)) / 2;
    const int m = 16 * br, ra = 16 * br + n, ib = 16 * bi + n;
    f32x4 ap = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int j = 32 * ks + 8 * g;
      float kt[8], qt[8], kh[8];
      bf8(Ks + ra * LDH + j, kt);
      bf8(Qs + ra * LDH + j, qt);
      bf8(Ks + ib * LDH + j, kh);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gm = Gs[m * LD + j + e];
        const float fr = exp2_raw(Gs[ra * LD + j + e] - gm);
        kt[e] *= fr;
        qt[e] *= fr;
        kh[e] *= exp2_raw(gm - Gs[ib * LD + j + e]);
      }
      bf16x8 kth, ktl, qth, qtl, khh, khl;
      split8(kt, kth, ktl);
      split8(qt, qth, qtl);
      split8(kh, khh, khl);
      aa = mfma_split3(kth, ktl, khh, khl, aa);
      ap = mfma_split3(qth, qtl, khh, khl, ap);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      put_split(Pc, C * C, (16 * br + 4 * g + e) * C + 16 * bi + n, ap[e]);
  } else {
    // The pairs (r, i), i <= r, inside the diagonal tiles, in groups of four:
    // rows r1 = 16 b + 2 u and r1 + 1 against columns i1 = 16 b + 2 v and
    // i1 + 1 (v <= u: 36 groups per tile; the pair (r1, i1 + 1) of a group
    // on the diagonal, v = u, lies above it and is dropped).  Four lanes
    // share a group, each summing every fourth slice of 2 dimensions, so
    // the K and Q rows are unpacked once for four pairs, and row r1 + 1's
    // factors come from row r1's:  e^{g_{r1+1} - g_i} = e^{g_{r1} - g_i} e^{g_{r1+1} - g_{r1}}.
    const int pidx = t - 6 * 64, quarter = pidx & 3, grp = pidx >> 2;
    if (grp < 4 * 36) {
      const int b = grp / 36, gg = grp % 36;
      int u = 0;
      while ((u + 1) * (u + 2) / 2 <= gg) ++u;
      const int v = gg - u * (u + 1) / 2;
      const int r1 = 16 * b + 2 * u, i1 = 16 * b + 2 * v;
      const uint16_t *kr1 = Ks + r1 * LDH, *qr1 = Qs + r1 * LDH, *ki1 = Ks + i1 * LDH;
      const float* g1p = Gs + r1 * LD;
      const float* h1p = Gs + i1 * LD;
      float a11 = 0.f, a12 = 0.f, a21 = 0.f, a22 = 0.f, p11 = 0.f, p12 = 0.f, p21 = 0.f, p22 = 0.f;
      auto dim = [&](float g1e, float g2e, float h1e, float h2e, float k1e, float k2e, float q1e,
                     float q2e, float c1e, float c2e) {
        const float sd = exp2_raw(g2e - g1e);
        const float e11 = exp2_raw(g1e - h1e) * c1e, e12 = exp2_raw(g1e - h2e) * c2e;
        const float e21 = e11 * sd, e22 = e12 * sd;
        a11 += k1e * e11, p11 += q1e * e11;
        a12 += k1e * e12, p12 += q1e * e12;
        a21 += k2e * e21, p21 += q2e * e21;
        a22 += k2e * e22, p22 += q2e * e22;
      };
      auto lo = [](uint32_t x) { return __uint_as_float(x << 16); };
      auto hi = [](uint32_t x) { return __uint_as_float(x & 0xffff0000u); };
#pragma unroll 1
      for (int m = 0; m < DK / 8; ++m) {  // 2-dimension slices 4 m + quarter
        const int j = 2 * (4 * m + quarter);
        const float2 g1 = *reinterpret_cast<const float2*>(g1p + j);
        const float2 g2 = *reinterpret_cast<const float2*>(g1p + LD + j);
        const float2 h1 = *reinterpret_cast<const float2*>(h1p + j);
        const float2 h2 = *reinterpret_cast<const float2*>(h1p + LD + j);
        const uint32_t k1 = *reinterpret_cast<const uint32_t*>(kr1 + j);
        const uint32_t k2 = *reinterpret_cast<const uint32_t*>(kr1 + LDH + j);
        const uint32_t q1 = *reinterpret_cast<const uint32_t*>(qr1 + j);
        const uint32_t q2 = *reinterpret_cast<const uint32_t*>(qr1 + LDH + j);
        const uint32_t c1 = *reinterpret_cast<const uint32_t*>(ki1 + j);
        const uint32_t c2 = *reinterpret_cast<const uint32_t*>(ki1 + LDH + j);
        dim(g1.x, g2.x, h1.x, h2.x, lo(k1), lo(k2), lo(q1), lo(q2), lo(c1), lo(c2));
        dim(g1.y, g2.y, h1.y, h2.y, hi(k1), hi(k2), hi(q1), hi(q2), hi(c1), hi(c2));
      }
      float sums[8] = {a11, p11, a21, p21, a22, p22, a12, p12};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sums[e] += __shfl_xor(sums[e], 1, 64);
        sums[e] += __shfl_xor(sums[e], 2, 64);
      }
      // Lane `quarter` keeps pair (r1, i1), (r1+1, i1), (r1+1, i1+1) or (r1, i1+1).
      const int r = r1 + (quarter == 1 || quarter == 2), i = i1 + (quarter >= 2);
      const float av_ = quarter == 0 ? sums[0] : quarter == 1 ? sums[2] : quarter == 2 ? sums[4] : sums[6];
      const float pv = quarter == 0 ? sums[1] : quarter == 1 ? sums[3] : quarter == 2 ? sums[5] : sums[7];
      if (i <= r) {
        put_split(Pc, C * C, r * C + i, pv);
        ar = r, ai = i;
        a = i < r ? av_ * bs[r] : 0.f;
      }
    }
  }
  __syncthreads();  // K and Q are dead from here: A goes over them
  if (w < 6) {
    const int br = w < 1 ? 1 : w < 3 ? 2 : 3;
    const int bi = w - (br * (br - 1)) / 2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * br + 4 * g + e;
      As[r * LDA + 16 * bi + n] = bs[r] * aa[e];
    }
  } else {  // (lanes without a pair write the zero diagonal entry (0, 0))
    As[ar * LDA + ai] = a;
  }

  // X = (I + A)^{-1} over the g tile (no longer needed), then T = X diag(beta).
  float* Xs = Gs;
  inv64::inverse<LDA, LD>(As, Xs, scratch);
  for (int e8 = t; e8 < C * C / 8; e8 += PNTHR) {
    const int r = e8 / (C / 8), i0 = 8 * (e8 % (C / 8));
    float tv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) tv[i] = Xs[r * LD + i0 + i] * bs[i0 + i];
    put_split8(Tc, C * C, 8 * e8, tv);
  }
}

template <int DK>
struct ScanLds {
  static constexpr int PK = DK + 8;
  static constexpr int PV = NT + 1;
  static constexpr size_t halves =
      2 * (size_t)DK * PC + 2 * (size_t)NT * PK + 4 * (size_t)NT * PC;
  static constexpr size_t bytes = halves * 2 + ((size_t)C * PV + DK) * sizeof(float);
};

template <typename OT> __device__ __forceinline__ void put_out(OT* p, float x);
template <> __device__ __forceinline__ void put_out<float>(float* p, float x) { *p = x; }
template <> __device__ __forceinline__ void put_out<bf16>(bf16* p, float x) { *p = from_f32<bf16>(x); }

template <int DK, int DV, typename OT>
__global__ __launch_bounds__(SNTH) void scan_kernel(const bf16* __restrict__ v,
                                                    const float* __restrict__ S0,
                                                    OT* __restrict__ o,
                                                    float* __restrict__ S_final, int L, int nc,
                                                    int nbh, const float* __restrict__ ws) {
  using LD = ScanLds<DK>;
  constexpr int PK = LD::PK, PV = LD::PV;
  constexpr int TPW = DK / 64;              // state row tiles per chain wave
  constexpr int KS = DK / 32;               // contraction steps over d_k
  constexpr int NKU = C * DK / 4 / NTH;     // float4 of K o e^{g_C - g} per chain thread
  static_assert(NKU == 4 || NKU == 8, "rows per thread");
  constexpr size_t CF = chunk_floats(DK);
  extern __shared__ uint4 lds_u4[];
  uint16_t* Uh = reinterpret_cast<uint16_t*>(lds_u4);  // (K o e^{g_C-g})^T, swizzled [DK][PC]
  uint16_t* Ul = Uh + DK * PC;
  uint16_t* Sh = Ul + DK * PC;                          // -S^T        [NT][PK]
  uint16_t* Sl = Sh + NT * PK;
  uint16_t* Rh = Sl + NT * PK;                          // R^T         [NT][PC]
  uint16_t* Rl = Rh + NT * PC;
  uint16_t* Dh = Rl + NT * PC;                          // Delta^T     [NT][PC]
  uint16_t* Dl = Dh + NT * PC;
  float* Vs = reinterpret_cast<float*>(Dl + NT * PC);   // V slice     [C][PV]
  float* gs = Vs + C * PV;                              // e^{g_C}     [DK]

  // 1-D grid of 8 * (d_v / 16) * ceil(nbh / 8): all column slices of a head
  // get the same flat id mod 8, so they share an XCD and its L2 (the
  // workspace block of a chunk is read by every slice).
  const int flat = blockIdx.x, xcd = flat & 7, sl = flat >> 3;
  const int j0 = (sl % (DV / NT)) * NT, bh = (sl / (DV / NT)) * 8 + xcd;
  if (bh >= nbh) return;
  const int t = threadIdx.x, l = t & 63, n = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  // Waves 0-3 carry the chain (R, Delta, the state); waves 4-7 form the
  // outputs.  Wave w of either kind owns chunk rows 16 (w & 3) .. + 15.
  const bool chain = w < 4;
  const int ct = t & (NTH - 1), r0 = 16 * (w & 3);
  const int ku_c4 = ct % (DK / 4), ku_r0 = NKU * (ct / (DK / 4));

  f32x4 S[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int d0 = 16 * ((w & 3) * TPW + i) + 4 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[i][e] = S0 && chain ? S0[((size_t)bh * DK + d0 + e) * DV + j0 + n] : 0.f;
  }

  // Next chunk's operands, in registers: (hi, lo) bf16 fragments straight
  // from the split planes of the workspace; phase 0 moves them into the
  // current chunk's set.  A chain wave holds rows of K o e^g and T (and its
  // share of K o e^{g_C - g}, v and e^{g_C}), an output wave rows of Q o e^g
  // and P, in the same registers.
  bf16x8 nah[KS], nal[KS], nbh_[2], nbl[2];
  uint2 kuh[NKU], kul[NKU];
  uint2 pv = make_uint2(0u, 0u);
  float pg = 0.f;
  auto fetch = [&](int cc) {
    const int vc = min(C, L - cc * C);
    const size_t t0 = (size_t)bh * L + (size_t)cc * C;
    const uint16_t* b = reinterpret_cast<const uint16_t*>(ws + ((size_t)bh * nc + cc) * CF);
    const uint16_t *bt = b, *bp = b + 2 * C * C, *bk = bp + 2 * C * C;
    const uint16_t *bq = bk + 2 * C * DK, *bu = bq + 2 * C * DK;
    const int row = r0 + n;
    auto ld16 = [](const uint16_t* p) { return as_bf16x8(*reinterpret_cast<const uint4*>(p)); };
    const uint16_t* ba = chain ? bk : bq;  // K o e^g or Q o e^g
    const uint16_t* bb = chain ? bt : bp;  // T or P
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = row * DK + 32 * ks + 8 * g;
      nah[ks] = ld16(ba + off);
      nal[ks] = ld16(ba + C * DK + off);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks > (w & 3) / 2) continue;  // T and P are lower triangular
      const int off = row * C + 32 * ks + 8 * g;
      nbh_[ks] = ld16(bb + off);
      nbl[ks] = ld16(bb + C * C + off);
    }
    if (chain) {
#pragma unroll
      for (int p = 0; p < NKU; ++p) {  // NKU consecutive rows of one 4-column group
        const int off = (ku_r0 + p) * DK + 4 * ku_c4;
        kuh[p] = *reinterpret_cast<const uint2*>(bu + off);
        kul[p] = *reinterpret_cast<const uint2*>(bu + C * DK + off);
      }
      const int r = ct % C, c4 = ct / C;
      const uint2 x =
          *reinterpret_cast<const uint2*>(v + (t0 + min(r, vc - 1)) * DV + j0 + 4 * c4);
      pv = r < vc ? x : make_uint2(0u, 0u);
      if (ct < DK) pg = reinterpret_cast<const float*>(bu + 2 * C * DK)[ct];
    }
  };

  // L2 prefetch of chunk c + 2: the 128-byte lines of its workspace block
  // and v rows are split over the head's column-slice workgroups (which
  // share an XCD); thread t touches line slice + NS t with one dword load.
  // The value is folded in a chunk later, so the load never stalls anything,
  // and the fold is only ever stored under a condition that is false.
  constexpr int NS = DV / NT;
  constexpr int WL = (int)(CF * 4 / 128), VL = C * DV * 2 / 128;
  constexpr int NPF = ((WL + VL + NS - 1) / NS + SNTH - 1) / SNTH;
  const int sidx = sl % NS;
  uint32_t pf_acc = 0, pf_val[NPF];
#pragma unroll
  for (int j = 0; j < NPF; ++j) pf_val[j] = 0;
  auto prefetch = [&](int cc) {
    const int vc = min(C, L - cc * C);
    const size_t t0 = (size_t)bh * L + (size_t)cc * C;
#pragma unroll
    for (int j = 0; j < NPF; ++j) {
      const int ln = min(sidx + NS * (t + SNTH * j), WL + VL - 1);
      const uint32_t* src;
      if (ln < WL) {
        src = reinterpret_cast<const uint32_t*>(ws + ((size_t)bh * nc + cc) * CF) + 32 * ln;
      } else {
        const int e = (ln - WL) * 64, row = min(e / DV, vc - 1);
        src = reinterpret_cast<const uint32_t*>(v + (t0 + row) * DV + e % DV);
      }
      pf_val[j] = *src;
    }
  };

  if (nc > 0) fetch(0);
  for (int c = 0; c < nc; ++c) {
    const int valid = min(C, L - c * C);
    const size_t tok0 = (size_t)bh * L + (size_t)c * C;
#pragma unroll
    for (int j = 0; j < NPF; ++j) pf_acc ^= pf_val[j];
    // Phase 0: this chunk's operands from the registers into split
    // fragments; the chain waves also stage K o e^{g_C - g} (transposed), the
    // v slice, e^{g_C} and the entering state in LDS.
    bf16x8 ah[KS], al[KS], bh2[2], bl2[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ah[ks] = nah[ks], al[ks] = nal[ks];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) bh2[ks] = nbh_[ks], bl2[ks] = nbl[ks];
    if (chain) {
      {  // (K o e^{g_C - g})^T: one NKU-row write per column and half
        uint32_t h[NKU][2], lo[NKU][2];
#pragma unroll
        for (int p = 0; p < NKU; ++p)
          h[p][0] = kuh[p].x, h[p][1] = kuh[p].y, lo[p][0] = kul[p].x, lo[p][1] = kul[p].y;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t ph[NKU / 2], pl[NKU / 2];
#pragma unroll
          for (int q = 0; q < NKU / 2; ++q) {
            const int sh = 16 * (e & 1);
            ph[q] = ((h[2 * q][e >> 1] >> sh) & 0xffffu) | ((h[2 * q + 1][e >> 1] >> sh) << 16);
            pl[q] = ((lo[2 * q][e >> 1] >> sh) & 0xffffu) | ((lo[2 * q + 1][e >> 1] >> sh) << 16);
          }
          const int off = tpos<2>(4 * ku_c4 + e, ku_r0);
          if constexpr (NKU == 8) {
            *reinterpret_cast<uint4*>(Uh + off) = make_uint4(ph[0], ph[1], ph[2], ph[3]);
            *reinterpret_cast<uint4*>(Ul + off) = make_uint4(pl[0], pl[1], pl[2], pl[3]);
          } else {
            *reinterpret_cast<uint2*>(Uh + off) = make_uint2(ph[0], ph[1]);
            *reinterpret_cast<uint2*>(Ul + off) = make_uint2(pl[0], pl[1]);
          }
        }
      }
      {
        const int r = ct % C, c4 = ct / C;
        Vs[r * PV + 4 * c4 + 0] = __uint_as_float(pv.x << 16);
        Vs[r * PV + 4 * c4 + 1] = __uint_as_float(pv.x & 0xffff0000u);
        Vs[r * PV + 4 * c4 + 2] = __uint_as_float(pv.y << 16);
        Vs[r * PV + 4 * c4 + 3] = __uint_as_float(pv.y & 0xffff0000u);
      }
      if (ct < DK) gs[ct] = pg;
#pragma unroll
      for (int i = 0; i < TPW; ++i) put_split_t(Sh, Sl, PK, 16 * ((w & 3) * TPW + i), -S[i]);
    }
    __syncthreads();
    if (c + 1 < nc) fetch(c + 1);
    prefetch(min(c + 2, nc - 1));

    // Phase 1: chain waves R = V - (K o e^g) S, output waves (Q o e^g)(-S);
    // row tile w & 3 each.
    f32x4 acc = zero4();
    if (chain) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = Vs[(r0 + 4 * g + e) * PV + n];
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = mfma_split3(ah[ks], al[ks], frag(Sh, PK, 0, 32 * ks), frag(Sl, PK, 0, 32 * ks), acc);
    if (chain) put_split_t(Rh, Rl, PC, r0, acc);
    __syncthreads();

    // Phase 2: Delta = T R, row tile w (T is lower triangular).
    if (chain) {
      f32x4 ad = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        if (ks <= (w & 3) / 2)
          ad = mfma_split3(bh2[ks], bl2[ks], frag(Rh, PC, 0, 32 * ks), frag(Rl, PC, 0, 32 * ks), ad);
      put_split_t(Dh, Dl, PC, r0, ad);
    }
    __syncthreads();

    // Phase 3: output waves O = (Q o e^g) S + P Delta (row tile w & 3); chain
    // waves S' = diag(e^{g_C}) S + (K o e^{g_C - g})^T Delta.
    if (!chain) {
      f32x4 ao = -acc;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        if (ks <= (w & 3) / 2)
          ao = mfma_split3(bh2[ks], bl2[ks], frag(Dh, PC, 0, 32 * ks), frag(Dl, PC, 0, 32 * ks), ao);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r0 + 4 * g + e;
        if (r < valid) put_out<OT>(o + (tok0 + r) * DV + j0 + n, ao[e]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int d0 = 16 * ((w & 3) * TPW + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) S[i][e] *= gs[d0 + 4 * g + e];
#pragma unroll
        for (int ks = 0; ks < C / 32; ++ks)
          S[i] = mfma_split3(fragT<2>(Uh, d0, 32 * ks), fragT<2>(Ul, d0, 32 * ks),
                             frag(Dh, PC, 0, 32 * ks), frag(Dl, PC, 0, 32 * ks), S[i]);
      }
    }
    __syncthreads();
  }
  if (S_final && chain)
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int d0 = 16 * ((w & 3) * TPW + i) + 4 * g;
#pragma unroll
      for (int e = 0; e < 4; ++e) S_final[((size_t)bh * DK + d0 + e) * DV + j0 + n] = S[i][e];
    }
#pragma unroll
  for (int j = 0; j < NPF; ++j) pf_acc ^= pf_val[j];
  if (nc < 0) S_final[0] = __uint_as_float(pf_acc);
}

template <int DK, int DV, typename OT>
hipError_t scan_t(const void* v, const float* S0, void* o, float* S_final, int L, int nc, int bh,
                  const float* ws, hipStream_t s) {
  auto* kern = &scan_kernel<DK, DV, OT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)ScanLds<DK>::bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(8 * (DV / NT) * ((bh + 7) / 8)), dim3(SNTH), ScanLds<DK>::bytes, s,
                     static_cast<const bf16*>(v), S0, static_cast<OT*>(o), S_final, L, nc, bh, ws);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t scan_types(int out_dtype, const void* v, const float* S0, void* o, float* S_final, int L,
                      int nc, int bh, const float* ws, hipStream_t s) {
  return out_dtype == 1 ? scan_t<DK, DV, bf16>(v, S0, o, S_final, L, nc, bh, ws, s)
                        : scan_t<DK, DV, float>(v, S0, o, S_final, L, nc, bh, ws, s);
}

}  // namespace mf

hipError_t launch_scan_mfma(int d_k, int d_v, int out_dtype, const void* v, const float* S0,
                            void* o, float* S_final, int L, int nc, int bh, const float* ws,
                            hipStream_t stream) {
  if (d_k == 64 && d_v == 64)
    return mf::scan_types<64, 64>(out_dtype, v, S0, o, S_final, L, nc, bh, ws, stream);
  if (d_k == 64 && d_v == 128)
    return mf::scan_types<64, 128>(out_dtype, v, S0, o, S_final, L, nc, bh, ws, stream);
  if (d_k == 128 && d_v == 64)
    return mf::scan_types<128, 64>(out_dtype, v, S0, o, S_final, L, nc, bh, ws, stream);
  return mf::scan_types<128, 128>(out_dtype, v, S0, o, S_final, L, nc, bh, ws, stream);
}

hipError_t launch_prep_mfma(int d_k, const void* q, const void* k, const float* alpha,
                            const float* beta, int L, int nc, int bh, float* ws,
                            hipStream_t stream) {
  auto run = [&](auto* kern, size_t bytes) -> hipError_t {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(nc, bh), dim3(mf::PNTHR), bytes, stream,
                       static_cast<const bf16*>(q), static_cast<const bf16*>(k), alpha, beta, L,
                       ws);
    return hipGetLastError();
  };
  if (d_k == 64) return run(&mf::prep_kernel<64>, mf::PrepLds<64>::bytes);
  return run(&mf::prep_kernel<128>, mf::PrepLds<128>::bytes);
}

}  // namespace kda
}  // namespace dn
