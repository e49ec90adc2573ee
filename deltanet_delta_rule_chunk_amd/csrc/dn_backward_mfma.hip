// dn_backward_mfma.hip -- the backward's kernels on the gfx950 matrix cores,
// for bf16 q, k, v: the prep (M per 64-token chunk), the reverse state
// pass and the kernel of the chunk's C x C gradients and dQ, dK.  (The
// forward pass that fills X, S, R and Delta runs on the chunked forward's
// own prep and scan at 128-token chunks: dn_chunk_mfma.hip and
// dn_scan_mfma.hip, their backward forms.)
//
// The products are those of the vector-ALU kernels in dn_backward.hip (the
// chunk algebra is derived there), taken as 16 x 16 x 32 bf16 MFMAs with
// fp32 accumulation.  q and k are exact in bf16; every fp32 operand (the
// state gradient G', X, M, dO, Delta, dDelta, dR, R, S, dT, Y, W) is carried
// as a split (hi, lo) bf16 pair (dn_mfma.h), so each product keeps roughly
// fp32 accuracy.
//
// The reverse pass runs one 8-wave workgroup per (head, 16 columns of d_v),
// all column slices of a head on one XCD; waves 0-3 carry the chain, the
// slice of the state gradient in MFMA accumulators (wave w holds the
// d_k / 64 row tiles w * d_k / 64 ...), and waves 4-7 load and deposit the
// next chunk.  Each chunk step is three phases separated by barriers:
//   1  chain wave w forms row tile w (16 chunk rows) of the first product;
//   2  chain wave w forms row tile w of the second, while the other waves
//      form Q^T dO (it needs no chain result);
//   3  every chain wave advances its state tiles while the next chunk's
//      operands go into LDS (row-major and, where a product contracts over
//      chunk rows, transposed copies); the ones phase 3 itself reads are
//      double buffered.
// Each step starts by writing the state gradient out and publishing it to
// LDS as a split B operand.

// LDS operand arrays are bf16 with rows padded by 16 bytes (dn_lds64.h).  A
// fragment read `frag(a, P, r0, kb)` gives lane l the 8 contraction slots
// kb + 8 (l / 16) ... of row r0 + l % 16, which is the A layout of the MFMA
// and, for an array stored [column][contraction], also its B layout.

#include "dn_backward.h"
#include "dn_common.h"
#include "dn_lds64.h"
#include "dn_mfma.h"
#include "dn_valu_common.h"

namespace dn {
namespace bwd {
namespace mf {

constexpr int NTH = 256;  // 4 waves
using namespace lds64;

// bf16 element e (0..7) of 16 bytes.
__device__ __forceinline__ uint16_t elem8(const uint4& x, int e) {
  const uint32_t w = (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
  return static_cast<uint16_t>(w >> (16 * (e & 1)));
}

// Loads of one chunk's C x DK bf16 tile (q or k): each thread takes N
// consecutive rows of one 16-byte column chunk (consecutive lanes along a
// row, so a wave's load covers whole cache lines); rows at or past `valid`
// read as zero (the load itself is clamped to a valid row).  Holding N rows
// of a column lets the transposed copy store N rows per LDS write.
template <int DK, int NTHR = NTH>
struct RowTile {
  static constexpr int CPR = DK / 8;              // 16-byte chunks per row
  static constexpr int N = C * CPR / NTHR;        // rows per thread
  static_assert(N == 2 || N == 4, "rows per thread");
  uint4 x[N];
  int tid = threadIdx.x;  // the thread's index among the NTHR that share the tile
  __device__ __forceinline__ int row0() const { return N * (tid / CPR); }
  __device__ __forceinline__ int chunk() const { return tid % CPR; }
  __device__ __forceinline__ void load(const bf16* src, int valid) {
    const uint4* s = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int p = 0; p < N; ++p) {
      const int r = row0() + p;
      const uint4 v = s[min(r, valid - 1) * CPR + chunk()];
      x[p] = r < valid ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // Row-major copy [C][DK + 8].
  __device__ __forceinline__ void put_rows(uint16_t* dst) const {
#pragma unroll
    for (int p = 0; p < N; ++p)
      *reinterpret_cast<uint4*>(dst + (row0() + p) * (DK + 8) + 8 * chunk()) = x[p];
  }
  // Transposed copy [DK][PC], swizzled (SH = 3): one N-row write per column.
  __device__ __forceinline__ void put_cols(uint16_t* dst) const {
    const int r0 = row0();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t* d = dst + tpos<3>(8 * chunk() + e, r0);
      if constexpr (N == 4) {
        *reinterpret_cast<uint2*>(d) =
            make_uint2(elem8(x[0], e) | (uint32_t)elem8(x[1], e) << 16,
                       elem8(x[2], e) | (uint32_t)elem8(x[3], e) << 16);
      } else {
        *reinterpret_cast<uint32_t*>(d) = elem8(x[0], e) | (uint32_t)elem8(x[1], e) << 16;
      }
    }
  }
};

// bf16 element e (0..3) of 4 packed in 8 bytes.
__device__ __forceinline__ uint32_t elem4(const uint2& h, int e) {
  return ((e < 2 ? h.x : h.y) >> (16 * (e & 1))) & 0xffffu;
}

// Loads of one chunk's C x C fp32 block of the workspace (X or M): each
// thread takes 4 consecutive rows of one 16-byte column chunk.
struct SqTile {
  static constexpr int CPR = C / 4;
  static constexpr int N = C * CPR / NTH;  // 4
  float4 x[N];
  int tid = threadIdx.x;  // the thread's index among the NTH that share the tile
  __device__ __forceinline__ int row0() const { return N * (tid / CPR); }
  __device__ __forceinline__ int chunk() const { return tid % CPR; }
  __device__ __forceinline__ void load(const float* src) {
    const float4* s = reinterpret_cast<const float4*>(src);
#pragma unroll
    for (int p = 0; p < N; ++p) x[p] = s[(row0() + p) * CPR + chunk()];
  }  // Split, row-major [C][PC].
  __device__ __forceinline__ void put_rows(uint16_t* hi, uint16_t* lo) const {
#pragma unroll
    for (int p = 0; p < N; ++p) {
      uint2 h, o;
      split4(x[p], h, o);
      const int off = (row0() + p) * PC + 4 * chunk();
      *reinterpret_cast<uint2*>(hi + off) = h;
      *reinterpret_cast<uint2*>(lo + off) = o;
    }
  }
  // Split, transposed [C][PC] and swizzled (SH = 2): one 4-row write per
  // column and half.
  __device__ __forceinline__ void put_cols(uint16_t* hi, uint16_t* lo) const {
    uint2 h[N], o[N];
#pragma unroll
    for (int p = 0; p < N; ++p) split4(x[p], h[p], o[p]);
    const int r0 = row0();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int off = tpos<2>(4 * chunk() + e, r0);
      *reinterpret_cast<uint2*>(hi + off) = make_uint2(elem4(h[0], e) | elem4(h[1], e) << 16,
                                                       elem4(h[2], e) | elem4(h[3], e) << 16);
      *reinterpret_cast<uint2*>(lo + off) = make_uint2(elem4(o[0], e) | elem4(o[1], e) << 16,
                                                       elem4(o[2], e) | elem4(o[3], e) << 16);
    }
  }
};

// ---- prep: M = tril(Q K^T) --------------------------------------------------
// One 4-wave workgroup per (chunk, head): wave w forms row tile w of M from
// the q and k rows in LDS (exact bf16 products, fp32 sums).  (X = (I + A)^{-1}
// of every 64-token chunk comes from the forward pass's prep, which inverts
// the 128-token I + A whose diagonal 64-row blocks these are.)
template <int DK>
struct PrepLds {
  static constexpr int PK = DK + 8;
  static constexpr size_t bytes = 2 * (size_t)C * PK * 2;  // K and Q rows, ~35 KB at d_k = 128
};

template <int DK, int DV>
__global__ __launch_bounds__(NTH) void prep_kernel(const bf16* __restrict__ q,
                                                   const bf16* __restrict__ k, int L,
                                                   float* __restrict__ ws) {
  using LD = PrepLds<DK>;
  constexpr int PK = LD::PK;
  constexpr Ws W{DK, DV};
  extern __shared__ uint4 lds_u4[];
  uint16_t* Kb = reinterpret_cast<uint16_t*>(lds_u4);  // K rows [C][PK]
  uint16_t* Qb = Kb + C * PK;                           // Q rows [C][PK]
  const int c = blockIdx.x, bh = blockIdx.y, nc = gridDim.x;
  const int valid = min(C, L - c * C);
  const size_t tok0 = (size_t)bh * L + (size_t)c * C;
  float* blk = ws + ((size_t)bh * nc + c) * W.per_chunk();
  const int t = threadIdx.x, w = t >> 6, l = t & 63, n = l & 15, g = l >> 4;
  const int r0 = 16 * w;
  {
    RowTile<DK> tq, tk;
    tq.load(q + tok0 * DK, valid);
    tk.load(k + tok0 * DK, valid);
    tq.put_rows(Qb);
    tk.put_rows(Kb);
  }
  __syncthreads();
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    // gq: tile (ct, w) of K Q^T, i.e. M's tile (w, ct) transposed, so that
    // each lane holds 4 consecutive columns of one row of M and stores them
    // with one 16-byte write.
    f32x4 gq = zero4();
    if (ct <= w) {
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks)
        gq = mfma16(frag(Kb, PK, 16 * ct, 32 * ks), frag(Qb, PK, r0, 32 * ks), gq);
    }
    const int mr = r0 + n, mi = 16 * ct + 4 * g;  // M[mr][mi .. mi + 3]
    *reinterpret_cast<float4*>(blk + W.M() + mr * C + mi) =
        make_float4(mi <= mr ? gq[0] : 0.f, mi + 1 <= mr ? gq[1] : 0.f, mi + 2 <= mr ? gq[2] : 0.f,
                    mi + 3 <= mr ? gq[3] : 0.f);
  }
}

// The state passes' workgroups: a 1-D grid of 8 * ns * ceil(nbh / 8), where
// ns = d_v / 16 column slices per head.  Workgroups go to the 8 XCDs
// round-robin by flat id; all slices of a head get the same flat id mod 8,
// so they run on one XCD and its L2 serves their common q, k, X, M reads.
// Returns false for the padding workgroups past the last head.
__device__ __forceinline__ bool slice_of(int ns, int nbh, int& j0, int& bh) {
  const int flat = blockIdx.x, xcd = flat & 7, sl = flat >> 3;
  j0 = (sl % ns) * NT;
  bh = (sl / ns) * 8 + xcd;
  return bh < nbh;
}

inline dim3 slice_grid(int ns, int nbh) { return dim3(8 * ns * ((nbh + 7) / 8)); }

// ---- reverse state pass -----------------------------------------------------
template <int DK>
struct BwdLds {
  static constexpr int PK = DK + 8;
  static constexpr size_t halves = (size_t)C * PK + 4 * (size_t)DK * PC + 4 * (size_t)C * PC +
                                   2 * (size_t)NT * PK + 8 * (size_t)NT * PC;
  static constexpr size_t bytes = halves * 2 + (size_t)C * sizeof(float) + (size_t)DK * NT * sizeof(float);
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Three barriers per chunk, as in the forward pass: the next chunk (in
// reverse order) is deposited during phase 3, with Q^T, K^T and dO^T, which
// are still read in phases 2 and 3, double buffered.  Eight waves: waves 0-3
// carry the chain (the three phases' products, the exit gradient and the
// stores); waves 4-7 load the next chunk, prefetch the one after into L2,
// form the chunk's input-only Q^T dO for the chain's state update and
// deposit the next chunk into LDS, off the chain's path.
constexpr int BNTH = 2 * NTH;

template <int DK, int DV>
__global__ __launch_bounds__(BNTH) void bwd_scan_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const float* __restrict__ beta,
    const float* __restrict__ dO, const float* __restrict__ dS_final, float* __restrict__ dv,
    float* __restrict__ dS0, int L, int nc, int nbh, float* __restrict__ ws) {
  using LD = BwdLds<DK>;
  constexpr int PK = LD::PK;
  constexpr Ws W{DK, DV};
  constexpr int TPW = DK / 64;
  extern __shared__ uint4 lds_u4[];
  uint16_t* Kb = reinterpret_cast<uint16_t*>(lds_u4);  // K rows        [C][PK]
  uint16_t* Kt = Kb + C * PK;                           // K^T           [2][DK][PC]
  uint16_t* Qt = Kt + 2 * DK * PC;                      // Q^T           [2][DK][PC]
  uint16_t* Mh = Qt + 2 * DK * PC;                      // M^T           [C][PC]
  uint16_t* Ml = Mh + C * PC;
  uint16_t* Xh = Ml + C * PC;                           // X^T           [C][PC]
  uint16_t* Xl = Xh + C * PC;
  uint16_t* Gh = Xl + C * PC;                           // G'^T          [NT][PK]
  uint16_t* Gl = Gh + NT * PK;
  uint16_t* Oh = Gl + NT * PK;                          // dO^T          [2][hi, lo][NT][PC]
  uint16_t* Eh = Oh + 4 * NT * PC;                      // dDelta^T      [NT][PC]
  uint16_t* El = Eh + NT * PC;
  uint16_t* Fh = El + NT * PC;                          // -dR^T         [NT][PC]
  uint16_t* Fl = Fh + NT * PC;
  float* bs = reinterpret_cast<float*>(Fl + NT * PC);
  float* Js = bs + C;  // Q^T dO of the chunk, [DK / 4][NT][4] (4-row groups)

  int j0, bh;
  if (!slice_of(DV / NT, nbh, j0, bh)) return;
  const int l = threadIdx.x & 63, n = l & 15, g = l >> 4;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool chain = wid < 4;
  const int w = wid & 3;                 // a chain wave's row tile and state tiles
  const int t = threadIdx.x & (NTH - 1);  // index within the role (loads, deposits)

  f32x4 G[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int d0 = 16 * (w * TPW + i) + 4 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      G[i][e] = dS_final && chain ? dS_final[((size_t)bh * DK + d0 + e) * DV + j0 + n] : 0.f;
  }

  RowTile<DK> tq, tk;
  SqTile tm, tx;
  tq.tid = tk.tid = tm.tid = tx.tid = t;
  float4 pd;
  float pb = 0.f;
  auto fetch = [&](int cc) {
    const int vc = min(C, L - cc * C);
    const size_t t0 = (size_t)bh * L + (size_t)cc * C;
    const float* b = ws + ((size_t)bh * nc + cc) * W.per_chunk();
    tq.load(q + t0 * DK, vc);
    tk.load(k + t0 * DK, vc);
    tm.load(b + W.M());
    tx.load(b + W.X());
    const int r = t % C, c4 = t / C;
    const float4 x = *reinterpret_cast<const float4*>(dO + (t0 + min(r, vc - 1)) * DV + j0 + 4 * c4);
    pd = r < vc ? x : make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < C) pb = t < vc ? beta[t0 + t] : 0.f;
  };

  // The fetched chunk into LDS (its Q^T, K^T, dO^T into buffer bb).
  auto deposit = [&](int bb) {
    tk.put_rows(Kb);
    tk.put_cols(Kt + bb * DK * PC);
    tq.put_cols(Qt + bb * DK * PC);
    tm.put_cols(Mh, Ml);
    tx.put_cols(Xh, Xl);
    uint16_t* oh = Oh + bb * 2 * NT * PC;
    uint16_t* ol = oh + NT * PC;
    const int r = t % C, c4 = t / C;
    uint2 h, o;
    split4(pd, h, o);
    oh[(4 * c4 + 0) * PC + r] = static_cast<uint16_t>(h.x);
    oh[(4 * c4 + 1) * PC + r] = static_cast<uint16_t>(h.x >> 16);
    oh[(4 * c4 + 2) * PC + r] = static_cast<uint16_t>(h.y);
    oh[(4 * c4 + 3) * PC + r] = static_cast<uint16_t>(h.y >> 16);
    ol[(4 * c4 + 0) * PC + r] = static_cast<uint16_t>(o.x);
    ol[(4 * c4 + 1) * PC + r] = static_cast<uint16_t>(o.x >> 16);
    ol[(4 * c4 + 2) * PC + r] = static_cast<uint16_t>(o.y);
    ol[(4 * c4 + 3) * PC + r] = static_cast<uint16_t>(o.y >> 16);
    if (t < C) bs[t] = pb;
  };

  // L2 prefetch of chunk c - 2: the 128-byte lines of its q, k, M, X rows and
  // dO rows are split over the head's column-slice workgroups (which share an
  // XCD); thread t touches line slice + ns t with one dword load, folded in a
  // chunk later and only ever stored under a condition that is false.
  constexpr int NS = DV / NT;
  constexpr int QL = C * DK * 2 / 128, ML = C * C * 4 / 128, OL = C * DV * 4 / 128;
  constexpr int NLINES = 2 * QL + 2 * ML + OL;
  constexpr int NPF = ((NLINES + NS - 1) / NS + NTH - 1) / NTH;
  const int sidx = (j0 / NT);
  uint32_t pf_acc = 0, pf_val[NPF];
#pragma unroll
  for (int i = 0; i < NPF; ++i) pf_val[i] = 0;
  auto prefetch = [&](int cc) {
    const int vc = min(C, L - cc * C);
    const size_t t0 = (size_t)bh * L + (size_t)cc * C;
    const float* b = ws + ((size_t)bh * nc + cc) * W.per_chunk();
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int ln = min(sidx + NS * (t + NTH * i), NLINES - 1);
      const uint32_t* src;
      if (ln < 2 * QL) {
        const int e = (ln % QL) * 64, row = min(e / DK, vc - 1);
        src = reinterpret_cast<const uint32_t*>((ln < QL ? q : k) + (t0 + row) * DK + e % DK);
      } else if (ln < 2 * QL + 2 * ML) {
        const int m = ln - 2 * QL;
        src = reinterpret_cast<const uint32_t*>(b + (m < ML ? W.M() : W.X())) + 32 * (m % ML);
      } else {
        const int e = (ln - 2 * QL - 2 * ML) * 32, row = min(e / DV, vc - 1);
        src = reinterpret_cast<const uint32_t*>(dO + (t0 + row) * DV + e % DV);
      }
      pf_val[i] = *src;
    }
  };

  if (!chain) {
    fetch(nc - 1);
    deposit((nc - 1) & 1);
  }
  for (int c = nc - 1; c >= 0; --c) {
#pragma unroll
    for (int i = 0; i < NPF; ++i) pf_acc ^= pf_val[i];
    const int valid = min(C, L - c * C);
    const size_t tok0 = (size_t)bh * L + (size_t)c * C;
    float* blk = ws + ((size_t)bh * nc + c) * W.per_chunk();
    const int bb = c & 1;
    const uint16_t* Kc = Kt + bb * DK * PC;
    const uint16_t* Qc = Qt + bb * DK * PC;
    const uint16_t* Oc = Oh + bb * 2 * NT * PC;
    const uint16_t* Ocl = Oc + NT * PC;
    // The exit gradient: out to the workspace and into LDS.
    if (chain) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int d0 = 16 * (w * TPW + i);
        store_tile16(G[i], blk + W.G() + (size_t)d0 * DV + j0, DV);
        put_split_t(Gh, Gl, PK, d0, G[i]);
      }
    }
    __syncthreads();
    if (!chain) {
      if (c > 0) fetch(c - 1);
      prefetch(max(c - 2, 0));
    }

    // Phase 1: dDelta = M^T dO + K G', row tile w (M^T is upper triangular,
    // so the first product starts at the tile's first row).
    const int r0 = 16 * w;
    f32x4 acc = zero4();
    if (chain) {
#pragma unroll
    for (int ks = 0; ks < C / 32; ++ks)
      if (ks >= w / 2)
        acc = mfma_split3(fragT<2>(Mh, r0, 32 * ks), fragT<2>(Ml, r0, 32 * ks), frag(Oc, PC, 0, 32 * ks),
                          frag(Ocl, PC, 0, 32 * ks), acc);
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks)
      acc = mfma_split2(frag(Kb, PK, r0, 32 * ks), frag(Gh, PK, 0, 32 * ks), frag(Gl, PK, 0, 32 * ks),
                        acc);
    store_tile16(acc, blk + W.dD() + (size_t)r0 * DV + j0, DV);
    put_split_t(Eh, El, PC, r0, acc);
    }
    __syncthreads();

    // Phase 2: dR = diag(beta) X^T dDelta, row tile w; dv = dR.  The loader
    // waves meanwhile form J = Q^T dO of the chunk (input only) for phase 3.
    if (!chain) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int d0 = 16 * (w * TPW + i);
        f32x4 jt = zero4();
#pragma unroll
        for (int ks = 0; ks < C / 32; ++ks)
          jt = mfma_split2(fragT<3>(Qc, d0, 32 * ks), frag(Oc, PC, 0, 32 * ks), frag(Ocl, PC, 0, 32 * ks), jt);
        *reinterpret_cast<f32x4*>(Js + ((d0 / 4 + g) * NT + n) * 4) = jt;
      }
    }
    if (chain) {
    acc = zero4();
#pragma unroll
    for (int ks = 0; ks < C / 32; ++ks)
      if (ks >= w / 2)
        acc = mfma_split3(fragT<2>(Xh, r0, 32 * ks), fragT<2>(Xl, r0, 32 * ks), frag(Eh, PC, 0, 32 * ks),
                          frag(El, PC, 0, 32 * ks), acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= bs[r0 + 4 * g + e];
    store_tile16(acc, dv + (tok0 + r0) * DV + j0, DV, valid - r0);
    put_split_t(Fh, Fl, PC, r0, -acc);
    }
    __syncthreads();

    // Phase 3: G = G' + Q^T dO - K^T dR; meanwhile the next chunk goes into
    // LDS (K rows, M^T, X^T and beta were last read in phases 1 and 2).
    if (chain) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int d0 = 16 * (w * TPW + i);
      G[i] += *reinterpret_cast<const f32x4*>(Js + ((d0 / 4 + g) * NT + n) * 4);
#pragma unroll
      for (int ks = 0; ks < C / 32; ++ks)
        G[i] = mfma_split2(fragT<3>(Kc, d0, 32 * ks), frag(Fh, PC, 0, 32 * ks), frag(Fl, PC, 0, 32 * ks),
                           G[i]);
    }
    } else if (c > 0) {
      deposit((c - 1) & 1);
    }
  }
  if (dS0 && chain)
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int d0 = 16 * (w * TPW + i) + 4 * g;
#pragma unroll
      for (int e = 0; e < 4; ++e) dS0[((size_t)bh * DK + d0 + e) * DV + j0 + n] = G[i][e];
    }
#pragma unroll
  for (int i = 0; i < NPF; ++i) pf_acc ^= pf_val[i];
  if (nc < 0) dv[0] = __uint_as_float(pf_acc);
}

// ---- the chunk's C x C gradients and dQ, dK in one kernel ------------------
// One workgroup of d_k / 16 waves per (chunk, head), so that dM and W never
// make a round trip through HBM and every row of dO, Delta, dDelta, R and
// dR is read once.
//   passes over d_v, 32 columns each: dO, Delta, dDelta, R and -dR staged
//      split in LDS; the S and G' rows of the pass are each wave's own B
//      operands, loaded from the workspace straight into registers.  Per pass:
//        - the C x C products dM = tril(dO Delta^T), dT = tril(dDelta R^T):
//          wave w takes row tile w % 4; with eight waves the pair w, w + 4
//          splits its column tiles, 0-1 and 2-3;
//        - dQ += dO S^T, dK += Delta G'^T - dR S^T: every wave owns column
//          tile w (16 columns of d_k) of both outputs, for all four 16-row
//          tiles;
//   then dbeta_i = sum_a X_ai dT_ai; Y = X^T dX with dX = dT diag(beta) (both
//      operands gathered from fp32 LDS columns and split); dA = -Y X^T
//      (strictly lower) and W = diag(beta) dA; the Gram tiles K K^T (exact
//      bf16 products) give dbeta_r += sum_{i<r} dA_ri (k_r . k_i) -- the same
//      row and column tiles per wave as the C x C products; dM and W go into
//      LDS as fp32;
//   then over chunk rows: dQ += dM K,  dK += dM^T Q + (W + W^T) K, with dM and
//      W split per fragment, K and Q staged transposed.
// LDS (about 72 KB at d_k = 128, two workgroups per CU): the passes' staging,
// then X, dT/Y, beta and the K rows, then dM and W with K^T and Q^T.
template <int DK>
struct GradLds {
  static constexpr int HJ = 32;  // d_v columns per pass
  static constexpr int PJ = HJ + 8;
  static constexpr int PF = C + 4;
  static constexpr int PK = DK + 8;
  static constexpr size_t s1 = 10 * (size_t)C * PJ * 2;                   // five split operands
  static constexpr size_t s2 = 2 * (size_t)C * PF * sizeof(float) + 3 * (size_t)C * sizeof(float) +
                               (size_t)C * PK * 2;  // X, dT/Y, beta, dbeta, sums, K rows
  static constexpr size_t s3 = 2 * (size_t)C * PF * sizeof(float) + 2 * (size_t)DK * PC * 2;  // dM, W, K^T, Q^T
  static constexpr size_t m12 = s1 > s2 ? s1 : s2;
  static constexpr size_t bytes = m12 > s3 ? m12 : s3;
};

template <int DK, int DV>
__global__ __launch_bounds__(DK * 4) void grad_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const float* __restrict__ beta,
    const float* __restrict__ dO, const float* __restrict__ dv, float* __restrict__ dq,
    float* __restrict__ dk, float* __restrict__ dbeta, int L, const float* __restrict__ ws) {
  using LD = GradLds<DK>;
  constexpr int HJ = LD::HJ < DV ? LD::HJ : DV, PJ = LD::PJ, PF = LD::PF, PK = LD::PK;
  constexpr Ws W{DK, DV};
  constexpr int NTQ = DK * 4;
  static_assert(NTQ >= 4 * 64, "four waves for the C x C products");
  constexpr bool kPairs = NTQ >= 8 * 64;
  constexpr int NCW = kPairs ? 2 : 4;  // C x C column tiles per wave
  constexpr int KS = HJ / 32;
  extern __shared__ uint4 lds_u4[];
  const int c = blockIdx.x, bh = blockIdx.y, nc = gridDim.x;
  const int valid = min(C, L - c * C);
  const size_t tok0 = (size_t)bh * L + (size_t)c * C;
  const float* blk = ws + ((size_t)bh * nc + c) * W.per_chunk();
  const int t = threadIdx.x, l = t & 63, n = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int rt = w & 3, r0 = 16 * rt, half = kPairs ? w >> 2 : 0;
  auto ctile = [&](int j) { return kPairs ? 2 * half + j : j; };  // this wave's column tiles

  // ---- passes over d_v ----------------------------------------------------------
  f32x4 am[NCW], at[NCW], aq[4], ak[4];
#pragma unroll
  for (int j = 0; j < NCW; ++j) am[j] = at[j] = zero4();
#pragma unroll
  for (int i = 0; i < 4; ++i) aq[i] = ak[i] = zero4();
  {
    uint16_t* Oh = reinterpret_cast<uint16_t*>(lds_u4);  // dO
    uint16_t* Ol = Oh + C * PJ;
    uint16_t* Dh = Ol + C * PJ;                           // Delta
    uint16_t* Dl = Dh + C * PJ;
    uint16_t* Eh = Dl + C * PJ;                           // dDelta
    uint16_t* El = Eh + C * PJ;
    uint16_t* Rh = El + C * PJ;                           // R
    uint16_t* Rl = Rh + C * PJ;
    uint16_t* Fh = Rl + C * PJ;                           // -dR
    uint16_t* Fl = Fh + C * PJ;
    for (int h = 0; h < DV; h += HJ) {
      float4 sv[KS][2], gv[KS][2];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const size_t o = (size_t)(16 * w + n) * DV + h + 32 * ks + 8 * g;
        sv[ks][0] = *reinterpret_cast<const float4*>(blk + W.S() + o);
        sv[ks][1] = *reinterpret_cast<const float4*>(blk + W.S() + o + 4);
        gv[ks][0] = *reinterpret_cast<const float4*>(blk + W.G() + o);
        gv[ks][1] = *reinterpret_cast<const float4*>(blk + W.G() + o + 4);
      }
      if (h > 0) __syncthreads();  // the previous pass is done with the staging
#pragma unroll
      for (int p = 0; p < C * HJ / 4 / NTQ; ++p) {
        const int f = t + p * NTQ, r = f / (HJ / 4), c4 = f % (HJ / 4);
        const size_t wo = (size_t)r * DV + h + 4 * c4;
        const size_t go = (tok0 + min(r, valid - 1)) * DV + h + 4 * c4;
        float4 xo = *reinterpret_cast<const float4*>(dO + go);
        float4 xf = *reinterpret_cast<const float4*>(dv + go);
        const float4 xd = *reinterpret_cast<const float4*>(blk + W.D() + wo);
        const float4 xe = *reinterpret_cast<const float4*>(blk + W.dD() + wo);
        const float4 xr = *reinterpret_cast<const float4*>(blk + W.R() + wo);
        if (r >= valid) xo = xf = make_float4(0.f, 0.f, 0.f, 0.f);
        xf = make_float4(-xf.x, -xf.y, -xf.z, -xf.w);
        const int o = r * PJ + 4 * c4;
        uint2 hh, ll;
        split4(xo, hh, ll);
        *reinterpret_cast<uint2*>(Oh + o) = hh;
        *reinterpret_cast<uint2*>(Ol + o) = ll;
        split4(xd, hh, ll);
        *reinterpret_cast<uint2*>(Dh + o) = hh;
        *reinterpret_cast<uint2*>(Dl + o) = ll;
        split4(xe, hh, ll);
        *reinterpret_cast<uint2*>(Eh + o) = hh;
        *reinterpret_cast<uint2*>(El + o) = ll;
        split4(xr, hh, ll);
        *reinterpret_cast<uint2*>(Rh + o) = hh;
        *reinterpret_cast<uint2*>(Rl + o) = ll;
        split4(xf, hh, ll);
        *reinterpret_cast<uint2*>(Fh + o) = hh;
        *reinterpret_cast<uint2*>(Fl + o) = ll;
      }
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // The C x C products of row tile rt (column tiles above the diagonal
        // are zero and skipped).
        if (ctile(0) <= rt) {
          const bf16x8 oh = frag(Oh, PJ, r0, 32 * ks), ol = frag(Ol, PJ, r0, 32 * ks);
          const bf16x8 eh = frag(Eh, PJ, r0, 32 * ks), el = frag(El, PJ, r0, 32 * ks);
#pragma unroll
          for (int j = 0; j < NCW; ++j) {
            const int ct = ctile(j);
            if (ct > rt) continue;
            am[j] = mfma_split3(oh, ol, frag(Dh, PJ, 16 * ct, 32 * ks), frag(Dl, PJ, 16 * ct, 32 * ks),
                                am[j]);
            at[j] = mfma_split3(eh, el, frag(Rh, PJ, 16 * ct, 32 * ks), frag(Rl, PJ, 16 * ct, 32 * ks),
                                at[j]);
          }
        }
        // dQ += dO S^T, dK += Delta G'^T - dR S^T, column tile w.
        uint2 h0, l0, h1, l1;
        split4(sv[ks][0], h0, l0);
        split4(sv[ks][1], h1, l1);
        const bf16x8 sh = as_bf16x8(h0, h1), sl = as_bf16x8(l0, l1);
        split4(gv[ks][0], h0, l0);
        split4(gv[ks][1], h1, l1);
        const bf16x8 gh = as_bf16x8(h0, h1), gl = as_bf16x8(l0, l1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          aq[i] = mfma_split3(frag(Oh, PJ, 16 * i, 32 * ks), frag(Ol, PJ, 16 * i, 32 * ks), sh, sl, aq[i]);
          ak[i] = mfma_split3(frag(Dh, PJ, 16 * i, 32 * ks), frag(Dl, PJ, 16 * i, 32 * ks), gh, gl, ak[i]);
          ak[i] = mfma_split3(frag(Fh, PJ, 16 * i, 32 * ks), frag(Fl, PJ, 16 * i, 32 * ks), sh, sl, ak[i]);
        }
      }
    }
  }
  __syncthreads();

  // ---- dbeta, Y, dA, W ----------------------------------------------------------
  f32x4 wv[NCW];  // this wave's tiles of W
  {
    float* Xs = reinterpret_cast<float*>(lds_u4);  // X    [C][PF]
    float* Ts = Xs + C * PF;                        // dT   [C][PF], then Y
    float* Ys = Ts;
    float* bs = Ts + C * PF;
    float* dbs = bs + C;
    float* rsb = dbs + C;                                 // the partner waves' dbeta sums
    uint16_t* Kb = reinterpret_cast<uint16_t*>(rsb + C);  // K rows [C][PK]
    {
      RowTile<DK, NTQ> tk;
      tk.load(k + tok0 * DK, valid);
#pragma unroll
      for (int p = 0; p < C * C / 4 / NTQ; ++p) {
        const int f = t + p * NTQ, r = f / (C / 4), c4 = f % (C / 4);
        *reinterpret_cast<float4*>(Xs + r * PF + 4 * c4) =
            *reinterpret_cast<const float4*>(blk + W.X() + r * C + 4 * c4);
      }
      if (t < C) bs[t] = t < valid ? beta[tok0 + t] : 0.f;
      tk.put_rows(Kb);
    }
#pragma unroll
    for (int j = 0; j < NCW; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r0 + 4 * g + e, i = 16 * ctile(j) + n;
        Ts[r * PF + i] = i <= r ? at[j][e] : 0.f;
      }
    __syncthreads();
    if (t < C) {  // dbeta_i from T = X diag(beta)
      float s = 0.f;
      for (int a = t; a < C; ++a) s += Xs[a * PF + t] * Ts[a * PF + t];
      dbs[t] = s;
    }
    // Y = X^T dX: Y_ab = sum_{r >= a} X_ra dT_rb beta_b (held in registers
    // until every wave is done reading dT, then written over it).
    f32x4 yt[NCW];
#pragma unroll
    for (int j = 0; j < NCW; ++j) {
      f32x4& y = yt[j];
      y = zero4();
      const int a = r0 + n, b = 16 * ctile(j) + n;
      const float bb = bs[b];
#pragma unroll
      for (int ks = 0; ks < C / 32; ++ks) {
        if (ks < rt / 2) continue;
        float xa[8], xb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 32 * ks + 8 * g + e;
          xa[e] = Xs[r * PF + a];
          xb[e] = Ts[r * PF + b] * bb;
        }
        bf16x8 ah, al, bh_, bl;
        split8(xa, ah, al);
        split8(xb, bh_, bl);
        y = mfma_split3(ah, al, bh_, bl, y);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NCW; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) Ys[(r0 + 4 * g + e) * PF + 16 * ctile(j) + n] = yt[j][e];
    __syncthreads();
    // dA = -Y X^T (strictly lower), W = diag(beta) dA, and the dbeta row sums
    // against the Gram tiles.
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NCW; ++j) {
      const int ct = ctile(j);
      f32x4 acc = zero4(), gr = zero4();
      if (ct <= rt) {
#pragma unroll
        for (int ks = 0; ks < C / 32; ++ks) {
          if (ks > ct / 2) continue;
          const float* ya = Ys + (r0 + n) * PF + 32 * ks + 8 * g;
          const float* xb = Xs + (16 * ct + n) * PF + 32 * ks + 8 * g;
          float va[8], vb[8];
          *reinterpret_cast<float4*>(va) = *reinterpret_cast<const float4*>(ya);
          *reinterpret_cast<float4*>(va + 4) = *reinterpret_cast<const float4*>(ya + 4);
          *reinterpret_cast<float4*>(vb) = *reinterpret_cast<const float4*>(xb);
          *reinterpret_cast<float4*>(vb + 4) = *reinterpret_cast<const float4*>(xb + 4);
          bf16x8 ah, al, bh_, bl;
          split8(va, ah, al);
          split8(vb, bh_, bl);
          acc = mfma_split3(ah, al, bh_, bl, acc);
        }
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks)
          gr = mfma16(frag(Kb, PK, r0, 32 * ks), frag(Kb, PK, 16 * ct, 32 * ks), gr);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r0 + 4 * g + e, i = 16 * ct + n;
        const float da = i < r ? -acc[e] : 0.f;
        wv[j][e] = bs[r] * da;
        rs[e] += da * gr[e];
      }
    }
    // The row sums over the wave's column tiles, then over the wave pair.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) rs[e] += __shfl_xor(rs[e], off, 64);
    }
    if (half == 1 && n == 0)
#pragma unroll
      for (int e = 0; e < 4; ++e) rsb[r0 + 4 * g + e] = rs[e];
    __syncthreads();
    if (half == 0 && n == 0)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r0 + 4 * g + e;
        if (r < valid) dbeta[tok0 + r] = dbs[r] + rs[e] + (kPairs ? rsb[r] : 0.f);
      }
  }
  __syncthreads();  // X, dT/Y and the K rows are dead: dM and W go over them

  // ---- dQ += dM K, dK += dM^T Q + (W + W^T) K ------------------------------------
  {
    float* Ms = reinterpret_cast<float*>(lds_u4);             // dM [C][PF]
    float* Wm = Ms + C * PF;                                   // W  [C][PF]
    uint16_t* Kt = reinterpret_cast<uint16_t*>(Wm + C * PF);  // K^T
    uint16_t* Qt = Kt + DK * PC;                               // Q^T
#pragma unroll
    for (int j = 0; j < NCW; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r0 + 4 * g + e, i = 16 * ctile(j) + n;
        Ms[r * PF + i] = i <= r ? am[j][e] : 0.f;
        Wm[r * PF + i] = wv[j][e];
      }
    {
      RowTile<DK, NTQ> tq, tk;
      tq.load(q + tok0 * DK, valid);
      tk.load(k + tok0 * DK, valid);
      tq.put_cols(Qt);
      tk.put_cols(Kt);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int ks = 0; ks < C / 32; ++ks) {
        const int r = 16 * i + n, a0 = 32 * ks + 8 * g;
        float m[8], mt[8], ww[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          m[e] = Ms[r * PF + a0 + e];
          mt[e] = Ms[(a0 + e) * PF + r];
          ww[e] = Wm[r * PF + a0 + e] + Wm[(a0 + e) * PF + r];
        }
        bf16x8 mh, ml, th, tl, wh, wl;
        split8(m, mh, ml);
        split8(mt, th, tl);
        split8(ww, wh, wl);
        const bf16x8 bk = fragT<3>(Kt, 16 * w, 32 * ks), bq = fragT<3>(Qt, 16 * w, 32 * ks);
        aq[i] = mfma16(mh, bk, aq[i]);
        aq[i] = mfma16(ml, bk, aq[i]);
        ak[i] = mfma16(th, bq, ak[i]);
        ak[i] = mfma16(tl, bq, ak[i]);
        ak[i] = mfma16(wh, bk, ak[i]);
        ak[i] = mfma16(wl, bk, ak[i]);
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * i + 4 * g + e;
      if (r < valid) {
        const size_t o = (tok0 + r) * DK + 16 * w + n;
        dq[o] = aq[i][e];
        dk[o] = ak[i][e];
      }
    }
}

template <typename K>
static hipError_t set_lds(K* kernel, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int DK, int DV>
hipError_t bwd_t(const void* q, const void* k, const float* beta, const float* dO,
                 const float* dS_final, float* dv, float* dS0, int L, int nc, int bh, float* ws,
                 hipStream_t s) {
  auto* kern = &bwd_scan_kernel<DK, DV>;
  hipError_t e = set_lds(kern, BwdLds<DK>::bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, slice_grid(DV / NT, bh), dim3(BNTH), BwdLds<DK>::bytes, s,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k), beta, dO, dS_final,
                     dv, dS0, L, nc, bh, ws);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t grad_t(const void* q, const void* k, const float* beta, const float* dO,
                  const float* dv, float* dq, float* dk, float* dbeta, int L, int nc, int bh,
                  const float* ws, hipStream_t s) {
  auto* kern = &grad_kernel<DK, DV>;
  hipError_t e = set_lds(kern, GradLds<DK>::bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(nc, bh), dim3(DK * 4), GradLds<DK>::bytes, s,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k), beta, dO, dv, dq,
                     dk, dbeta, L, ws);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t prep_t(const void* q, const void* k, int L, int nc, int bh, float* ws, hipStream_t s) {
  auto* kern = &prep_kernel<DK, DV>;
  hipError_t e = set_lds(kern, PrepLds<DK>::bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(nc, bh), dim3(NTH), PrepLds<DK>::bytes, s,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k), L, ws);
  return hipGetLastError();
}

}  // namespace mf

hipError_t launch_bwd_scan_mfma(int d_k, int d_v, const void* q, const void* k,
                                const float* beta, const float* dO, const float* dS_final,
                                float* dv, float* dS0, int L, int nc, int bh, float* ws,
                                hipStream_t stream) {
  if (d_k == 64 && d_v == 64)
    return mf::bwd_t<64, 64>(q, k, beta, dO, dS_final, dv, dS0, L, nc, bh, ws, stream);
  if (d_k == 64 && d_v == 128)
    return mf::bwd_t<64, 128>(q, k, beta, dO, dS_final, dv, dS0, L, nc, bh, ws, stream);
  if (d_k == 128 && d_v == 64)
    return mf::bwd_t<128, 64>(q, k, beta, dO, dS_final, dv, dS0, L, nc, bh, ws, stream);
  return mf::bwd_t<128, 128>(q, k, beta, dO, dS_final, dv, dS0, L, nc, bh, ws, stream);
}

hipError_t launch_grad_mfma(int d_k, int d_v, const void* q, const void* k, const float* beta,
                            const float* dO, const float* dv, float* dq, float* dk,
                            float* dbeta, int L, int nc, int bh, const float* ws,
                            hipStream_t stream) {
  if (d_k == 64 && d_v == 64)
    return mf::grad_t<64, 64>(q, k, beta, dO, dv, dq, dk, dbeta, L, nc, bh, ws, stream);
  if (d_k == 64 && d_v == 128)
    return mf::grad_t<64, 128>(q, k, beta, dO, dv, dq, dk, dbeta, L, nc, bh, ws, stream);
  if (d_k == 128 && d_v == 64)
    return mf::grad_t<128, 64>(q, k, beta, dO, dv, dq, dk, dbeta, L, nc, bh, ws, stream);
  return mf::grad_t<128, 128>(q, k, beta, dO, dv, dq, dk, dbeta, L, nc, bh, ws, stream);
}

hipError_t launch_prep_mfma(int d_k, int d_v, const void* q, const void* k, int L, int nc, int bh,
                            float* ws, hipStream_t stream) {
  if (d_k == 64 && d_v == 64) return mf::prep_t<64, 64>(q, k, L, nc, bh, ws, stream);
  if (d_k == 64 && d_v == 128) return mf::prep_t<64, 128>(q, k, L, nc, bh, ws, stream);
  if (d_k == 128 && d_v == 64) return mf::prep_t<128, 64>(q, k, L, nc, bh, ws, stream);
  return mf::prep_t<128, 128>(q, k, L, nc, bh, ws, stream);
}

}  // namespace bwd
}  // namespace dn
