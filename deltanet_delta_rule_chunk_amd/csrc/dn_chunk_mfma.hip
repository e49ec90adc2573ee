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
// parallel, ~52 KB of LDS so three workgroups share a CU.  With 16 x 16
// tiles (NT = C / 16 tile rows):
//   1-2. k rows -> LDS (swizzled, dn_ktile.h) 64 columns of d_k at a time,
//      and the Gram tiles on bf16 MFMA accumulated over the slices (bf16
//      products are exact, sums fp32), the next slice's loads in flight
//      meanwhile.  The off-diagonal tiles of A are kept as split-bf16 MFMA
//      operands, the diagonal tiles' strictly lower parts N_i as fp32.
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
//
// Gated form (GATED; Gated DeltaNet, article "How a Baseten Engineer Traced 7
// Years of Attention Mechanism Evolution", Gated DeltaNet section: decay by
// alpha_t first, then the precise write).  Decaying the state before each
// write scales every pair (r, i), i < r, of the chunk by the decays between
// them, e^{g_r - g_i} with g_r = log(alpha_1) + ... + log(alpha_r):
//     A_ri = beta_r e^{g_r - g_i} (k_r . k_i),
// and T = (I + A)^{-1} diag(beta) as before.  The kernel also writes the g_r
// of the chunk (rows past L: alpha = 1) for the scan.

#include "dn_common.h"
#include "dn_features.h"
#include "dn_ktile.h"
#include "dn_launch.h"
#include "dn_mfma.h"
#include "dn_tfrag.h"

#include <type_traits>

namespace dn {

hipError_t launch_scan_mfma(const ChunkArgs& a, const uint4* Tfrag, const float* Gws);

namespace prep {

template <int C, int DK>
struct Cfg {
  static constexpr int NT = C / 16;                    // 16-row tiles
  static constexpr int KW = 64;                        // d_k columns staged at a time
  static constexpr int NH = DK / KW;                   // staging passes over d_k
  static constexpr int NOFF = NT * (NT - 1) / 2;       // off-diagonal lower tiles
  static constexpr int SPT = C * KW / (8 * 256);       // staged 16-byte k pieces per thread
  // LDS, in bytes.  Region 0 holds a C x 64 slice of the k tile, later the
  // two fp32 layouts of the diagonal inverses; ~52 KB in all, so three
  // workgroups share a CU.
  static constexpr int R0 = C * KW * 2 > NT * 2048 ? C * KW * 2 : NT * 2048;
  static constexpr int OFF_A = R0;                     // NOFF tiles x 2 planes x 512 B
  static constexpr int OFF_N = OFF_A + NOFF * 1024;    // NT tiles x 1 KB fp32
  static constexpr int OFF_BETA = OFF_N + NT * 1024;   // C floats
  static constexpr size_t bytes = (size_t)OFF_BETA + C * 4;
  static_assert(SPT >= 1, "shape");
};

// Gated form: the chunk's cumulative log-decays live in registers, lane l
// holding rows GE l .. GE l + GE - 1 (GE = C / 64); any row's value is fetched
// with a lane shuffle (every lane may ask for a different row).  Keeping them
// out of LDS keeps the LDS at a size where three workgroups share a CU.
template <int C>
struct GRegs {
  static constexpr int GE = C / 64;
  float v[GE];
  __device__ __forceinline__ float at(int row) const {
    if constexpr (GE == 1) {
      return __shfl(v[0], row, 64);
    } else {
      const float a = __shfl(v[0], row >> 1, 64), b = __shfl(v[1], row >> 1, 64);
      return (row & 1) ? b : a;
    }
  }
};

// Lower tile (i, k), i > k, of A: index in the off-diagonal list.
__device__ __forceinline__ int tidx(int i, int k) { return i * (i - 1) / 2 + k; }

__device__ __forceinline__ bf16x8 lds16(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(p));
}

// Gram tile columns of wave W: tile (i, kk), kk <= i, computed as
// K_kk K_i^T so that lane (i16, g) register r holds
// G[16 i + i16][16 kk + 4 g + r]: A_{i,kk} in row layout.  Columns
// kk = W and NT - 1 - W (NT + 1 tiles in all).  Each call adds the products
// over one 64-column slice of k (staged in Ks); the final call writes the
// off-diagonal tiles of A = diag(beta) G to Atl as split operands and the
// strictly lower part of the diagonal tile to Nd (fp32, column-major:
// Nd[i][col][row] = N_i[row][col]); in the gated form each element first
// takes its decay factor e^{g_row - g_col}.
template <int C, int W, bool FINAL, bool GATED>
__device__ __forceinline__ void gram_wave(const uint16_t* Ks, f32x4 (&acc)[2][C / 16], uint2* Atl,
                                          float* Nd, const float* bs, const GRegs<C>& gr_, int lane,
                                          int g, int i16) {
  constexpr int NT = C / 16, KW = 64, NKB = KW / 32;
  if constexpr (W < NT / 2) {
#pragma unroll
    for (int gc = 0; gc < 2; ++gc) {
      const int kk = gc == 0 ? W : NT - 1 - W;
      bf16x8 Ak[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) Ak[kb] = lds16(Ks + koff<KW>(16 * kk + i16, 4 * kb + g));
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if (i < kk) continue;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          acc[gc][i] = mfma16(Ak[kb], lds16(Ks + koff<KW>(16 * i + i16, 4 * kb + g)), acc[gc][i]);
      }
      if constexpr (FINAL) {
        float gcol[4];
        if constexpr (GATED) {
#pragma unroll
          for (int r = 0; r < 4; ++r) gcol[r] = gr_.at(16 * kk + 4 * g + r);
        }
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          if (i < kk) continue;
          const float b = bs[16 * i + i16];
          if constexpr (GATED) {  // e^{g_row - g_col}; only col <= row is kept
            const float grow = gr_.at(16 * i + i16);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[gc][i][r] *= __expf(fminf(grow - gcol[r], 0.f));
          }
          if (i > kk) {
            uint2 hi, lo;
            split4(acc[gc][i] * b, hi, lo);
            Atl[tidx(i, kk) * 128 + lane] = hi;
            Atl[tidx(i, kk) * 128 + 64 + lane] = lo;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int col = 4 * g + r;
              Nd[i * 256 + col * 16 + i16] = col < i16 ? acc[gc][i][r] * b : 0.f;
            }
          }
        }
      }
    }
  }
}

// Tile columns j = W and NT - 1 - W of T (waves W >= NT / 2 have none):
//     T_jj = Linv_j diag(beta_j),
//     T_ij = Linv_i R_ij,  R_ij = -sum_{j <= k < i} A_ik T_kj   (i > j),
// the two columns' row chains advancing together.  T_kj is kept split in
// column layout (lane (i16, g) holds T_kj[4 g + r][i16]), the B operand of
// the next rows; each T_ij is also formed transposed, R_ij^T Linv_i^T, which
// is its row layout, and stored as half of fragment block (i, j / 2).
// XOUT (C = 128, the forward pass of the backward): the chains carry
// X = (I + A)^{-1} instead (the same substitution without beta), T_ij =
// X_ij diag(beta_j) is formed for the store, and the tiles of X inside the
// two 64-row diagonal blocks go row-major in fp32 to xb0 and xb1 (null: no
// such block), the tiles above the diagonal as zeros.
template <int C, int W, bool XOUT>
__device__ __forceinline__ void cols_wave(const uint2* Atl, const float* Lrow, const float* Lcol,
                                          const float* bs, uint4* out, int lane, int g, int i16,
                                          float* xb0, float* xb1) {
  constexpr int NT = C / 16;
  static_assert(!XOUT || C == 128, "X blocks of a 128-row chunk");
  if constexpr (W < NT / 2) {
    constexpr int J[2] = {W, NT - 1 - W};
    auto tstore = [&](int i, int j, uint2 hi, uint2 lo) {
      uint2* blk = reinterpret_cast<uint2*>(out + (size_t)(Frag<C>::base(i) + j / 2) * 128);
      blk[2 * lane + (j & 1)] = hi;
      blk[128 + 2 * lane + (j & 1)] = lo;
    };
    // Row layout tile (i, j) of X into its 64-row block (lane (i16, g): row
    // i16, columns 4 g .. 4 g + 3).
    auto xstore = [&](int i, int j, f32x4 x) {
      float* xb = i < 4 ? xb0 : xb1;
      if ((i >> 2) == (j >> 2) && xb)
        *reinterpret_cast<f32x4*>(xb + (16 * (i & 3) + i16) * 64 + 16 * (j & 3) + 4 * g) = x;
    };
    const uint2 z = make_uint2(0u, 0u);
    uint2 th[2][NT], tl[2][NT];
#pragma unroll
    for (int cw = 0; cw < 2; ++cw) {
      const int j = J[cw];
#pragma unroll
      for (int t = 0; t < NT; ++t) { th[cw][t] = z; tl[cw][t] = z; }
      const f32x4 lc = *reinterpret_cast<const f32x4*>(Lcol + j * 256 + lane * 4);
      if constexpr (XOUT)
        split4(lc, th[cw][j], tl[cw][j]);
      else
        split4(lc * bs[16 * j + i16], th[cw][j], tl[cw][j]);
      const f32x4 lr = *reinterpret_cast<const f32x4*>(Lrow + j * 256 + lane * 4);
      const float4 brow = *reinterpret_cast<const float4*>(bs + 16 * j + 4 * g);
      f32x4 trow;
      trow[0] = lr[0] * brow.x; trow[1] = lr[1] * brow.y;
      trow[2] = lr[2] * brow.z; trow[3] = lr[3] * brow.w;
      uint2 hi, lo;
      split4(trow, hi, lo);
      tstore(j, j, hi, lo);
      if (j & 1) tstore(j - 1, j, z, z);
      if constexpr (XOUT) {
        xstore(j, j, lr);
#pragma unroll
        for (int i = 0; i < NT; ++i)
          if (i < j) xstore(i, j, zero4());
      }
    }
#pragma unroll
    for (int i = 1; i < NT; ++i) {
      const f32x4 lr = *reinterpret_cast<const f32x4*>(Lrow + i * 256 + lane * 4);
      uint2 lh, ll;
      split4(lr, lh, ll);
      const bf16x8 Lh = as_bf16x8(lh, z), Ll = as_bf16x8(ll, z);
#pragma unroll
      for (int cw = 0; cw < 2; ++cw) {
        const int j = J[cw];
        if (i <= j) continue;
        // R_ij = -sum_k A_ik T_kj over tile pairs (2p, 2p + 1); T_kj = 0 for
        // k < j and A_ik is only taken for k < i.
        f32x4 a0 = zero4(), a1 = zero4(), a2 = zero4();
#pragma unroll
        for (int p = 0; p < NT / 2; ++p) {
          if (2 * p > i - 1 || 2 * p + 1 < j) continue;
          const uint2 ah0 = Atl[tidx(i, 2 * p) * 128 + lane], al0 = Atl[tidx(i, 2 * p) * 128 + 64 + lane];
          const bool two = 2 * p + 1 < i;
          const uint2 ah1 = two ? Atl[tidx(i, 2 * p + 1) * 128 + lane] : z;
          const uint2 al1 = two ? Atl[tidx(i, 2 * p + 1) * 128 + 64 + lane] : z;
          const bf16x8 Ah = as_bf16x8(ah0, ah1), Al = as_bf16x8(al0, al1);
          const bf16x8 Bh = as_bf16x8(th[cw][2 * p], th[cw][2 * p + 1]);
          const bf16x8 Bl = as_bf16x8(tl[cw][2 * p], tl[cw][2 * p + 1]);
          a0 = mfma16(Ah, Bh, a0);
          a1 = mfma16(Ah, Bl, a1);
          a2 = mfma16(Al, Bh, a2);
        }
        const f32x4 R = -(a0 + a1 + a2);
        uint2 rh, rl;
        split4(R, rh, rl);
        const bf16x8 Rh = as_bf16x8(rh, z), Rl = as_bf16x8(rl, z);
        // T_ij = Linv_i R_ij (column layout, kept for the next rows).
        f32x4 tc = mfma16(Lh, Rh, zero4());
        tc = mfma16(Lh, Rl, tc);
        tc = mfma16(Ll, Rh, tc);
        split4(tc, th[cw][i], tl[cw][i]);
        // T_ij^T = R_ij^T Linv_i^T (row layout, stored).
        f32x4 tr = mfma16(Rh, Lh, zero4());
        tr = mfma16(Rh, Ll, tr);
        tr = mfma16(Rl, Lh, tr);
        if constexpr (XOUT) {  // tr is X_ij: store it, then T_ij = X_ij diag(beta_j)
          xstore(i, j, tr);
          const float4 brow = *reinterpret_cast<const float4*>(bs + 16 * j + 4 * g);
          tr[0] *= brow.x; tr[1] *= brow.y; tr[2] *= brow.z; tr[3] *= brow.w;
        }
        uint2 hi, lo;
        split4(tr, hi, lo);
        tstore(i, j, hi, lo);
      }
    }
  }
}

// FEAT: k and beta are the raw k projection and the beta logits; the
// layer's feature maps are applied as the rows arrive (the same arithmetic
// as the streaming feature kernel, so the same bits), and the mapped q, k
// and beta are written out for the scan.  q_raw, q_hat, k_hat and beta_out
// are used only then.  XOUT: the forward pass of the backward, which also
// takes X of each 64-token block into the backward's workspace (bo).
template <int C, int DK, bool GATED, bool FEAT, bool XOUT = false>
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ k,
                                                   const float* __restrict__ alpha,
                                                   const float* __restrict__ beta, int L,
                                                   int nc, uint4* __restrict__ Tfrag,
                                                   float* __restrict__ Gws,
                                                   const uint16_t* __restrict__ q_raw,
                                                   uint16_t* __restrict__ q_hat,
                                                   uint16_t* __restrict__ k_hat,
                                                   float* __restrict__ beta_out, BwdFwdOut bo) {
  static_assert(!XOUT || (C == 128 && !GATED && !FEAT), "the backward's forward pass");
  using CF = Cfg<C, DK>;
  constexpr int NT = CF::NT;
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

  // ---- 1-2. k tile (64 columns at a time) and Gram tiles -------------------
  // The next slice's loads are in flight while the current one is used.
  constexpr int KW = CF::KW, NH = CF::NH, SPT = CF::SPT;
  // With the feature maps the rows come whole (a row's norm needs all of
  // it): PPR adjacent lanes hold a row, 16 bytes each, FPT pieces per
  // thread; piece p of a row lies in staging slice p / (KW / 8).
  constexpr int PPR = DK / 8, FPT = C * DK / (8 * 256);
  static_assert(256 % PPR == 0 && FPT >= 1, "row pieces");
  uint4 kv[FEAT ? FPT : SPT];
  auto kload = [&](int h) {
    if constexpr (!FEAT) {
#pragma unroll
      for (int i = 0; i < SPT; ++i) {
        const int e = i * 256 + tid, row = e / (KW / 8), ch = e % (KW / 8);
        kv[i] = *reinterpret_cast<const uint4*>(k + (tok0 + min(row, valid - 1)) * DK + h * KW + ch * 8);
      }
    }
  };
  auto kstore = [&](int h) {
    if constexpr (FEAT) {
      const int p = tid % PPR;
      if (p / (KW / 8) == h) {
#pragma unroll
        for (int i = 0; i < FPT; ++i)
          *reinterpret_cast<uint4*>(Ks + koff<KW>((i * 256 + tid) / PPR, p % (KW / 8))) = kv[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < SPT; ++i) {
        const int e = i * 256 + tid, row = e / (KW / 8), ch = e % (KW / 8);
        const uint32_t m = row < valid ? 0xffffffffu : 0u;
        *reinterpret_cast<uint4*>(Ks + koff<KW>(row, ch)) =
            make_uint4(kv[i].x & m, kv[i].y & m, kv[i].z & m, kv[i].w & m);
      }
    }
  };
  if constexpr (FEAT) {
    // Raw q and k rows (rows past L as zeros, which map to zeros), mapped;
    // the mapped rows of the sequence go to the workspace.
    using feat::u32x4;
    const int p = tid % PPR;
    uint4 qv[FPT];
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
      const int row = (i * 256 + tid) / PPR;
      const size_t off = (tok0 + min(row, valid - 1)) * DK + 8 * p;
      const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + off));
      const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q_raw + off));
      const bool in = row < valid;
      kv[i] = in ? make_uint4(a.x, a.y, a.z, a.w) : make_uint4(0u, 0u, 0u, 0u);
      qv[i] = in ? make_uint4(b.x, b.y, b.z, b.w) : make_uint4(0u, 0u, 0u, 0u);
    }
    const float bl = tid < valid && tid < C ? beta[tok0 + tid] : 0.f;
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
      const int row = (i * 256 + tid) / PPR;
      kv[i] = feat::map_piece<PPR, 8>(kv[i]);
      const uint4 qm = feat::map_piece<PPR, 8>(qv[i]);
      if (row < valid) {
        const size_t off = (tok0 + row) * DK + 8 * p;
        __builtin_nontemporal_store(u32x4{kv[i].x, kv[i].y, kv[i].z, kv[i].w},
                                    reinterpret_cast<u32x4*>(k_hat + off));
        __builtin_nontemporal_store(u32x4{qm.x, qm.y, qm.z, qm.w},
                                    reinterpret_cast<u32x4*>(q_hat + off));
      }
    }
    if (tid < C) {
      const float b = tid < valid ? fast_sigmoid(bl) : 0.f;
      bs[tid] = b;
      if (tid < valid) beta_out[tok0 + tid] = b;
    }
  } else {
    kload(0);
    if (tid < C) bs[tid] = tid < valid ? beta[tok0 + tid] : 0.f;
  }
  // Gated form: g_r by an inclusive scan over each wave (every wave keeps its
  // own copy in registers); wave 0 also writes the chunk's g to the workspace.
  GRegs<C> gr_;
  if constexpr (GATED) {
    constexpr int E = GRegs<C>::GE;
    float run = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int r = E * lane + e;
      gr_.v[e] = r < valid ? log_decay(alpha[tok0 + r]) : 0.f;
      run += gr_.v[e];
    }
    float x = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float t = __shfl_up(x, off, 64);
      if (lane >= off) x += t;
    }
    float pre = x - run;
#pragma unroll
    for (int e = 0; e < E; ++e) gr_.v[e] = pre += gr_.v[e];
    if (w == 0) {
      float* const gout = Gws + ((size_t)bh * nc + c) * C;
#pragma unroll
      for (int e = 0; e < E; ++e) gout[E * lane + e] = gr_.v[e];
    }
  }
  kstore(0);
  f32x4 acc[2][NT];
#pragma unroll
  for (int gc = 0; gc < 2; ++gc)
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[gc][i] = zero4();
  // Wave w owns the Gram tile columns kk = w and kk = NT - 1 - w; the wave
  // index is made a compile-time constant so every loop below is static and
  // the compiler can interleave the independent tiles.
  auto gram = [&](auto final_tag) {
    constexpr bool F = decltype(final_tag)::value;
    switch (w) {
      case 0: gram_wave<C, 0, F, GATED>(Ks, acc, Atl, Nd, bs, gr_, lane, g, i16); break;
      case 1: gram_wave<C, 1, F, GATED>(Ks, acc, Atl, Nd, bs, gr_, lane, g, i16); break;
      case 2: gram_wave<C, 2, F, GATED>(Ks, acc, Atl, Nd, bs, gr_, lane, g, i16); break;
      default: gram_wave<C, 3, F, GATED>(Ks, acc, Atl, Nd, bs, gr_, lane, g, i16); break;
    }
  };
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    if (h + 1 < NH) kload(h + 1);
    __syncthreads();
    if (h + 1 < NH) {
      gram(std::integral_constant<bool, false>{});
      __syncthreads();
      kstore(h + 1);
    } else {
      gram(std::integral_constant<bool, true>{});
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
  float *xb0 = nullptr, *xb1 = nullptr;
  if constexpr (XOUT) {  // blocks 2c and 2c + 1 (the latter only if it exists)
    xb0 = bo.ws + ((size_t)bh * bo.nb + 2 * c) * bo.block + bo.x;
    if (2 * c + 1 < bo.nb) xb1 = xb0 + bo.block;
  }
  switch (w) {
    case 0: cols_wave<C, 0, XOUT>(Atl, Lrow, Lcol, bs, out, lane, g, i16, xb0, xb1); break;
    case 1: cols_wave<C, 1, XOUT>(Atl, Lrow, Lcol, bs, out, lane, g, i16, xb0, xb1); break;
    case 2: cols_wave<C, 2, XOUT>(Atl, Lrow, Lcol, bs, out, lane, g, i16, xb0, xb1); break;
    default: cols_wave<C, 3, XOUT>(Atl, Lrow, Lcol, bs, out, lane, g, i16, xb0, xb1); break;
  }
}

template <int C, int DK, bool GATED, bool FEAT, bool XOUT = false>
hipError_t launch_g(const ChunkArgs& a, uint4* Tfrag, float* Gws) {
  const int nc = cdiv(a.L, C);
  const int BH = a.B * a.H;
  constexpr size_t sm = Cfg<C, DK>::bytes;
  auto* kern = &prep_kernel<C, DK, GATED, FEAT, XOUT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  const FeatureArgs* f = a.feat;
  if (!a.bwd_out) prof_mark(kSlotChunkPrep, false, a.stream);
  hipLaunchKernelGGL(kern, dim3(nc, BH), dim3(256), sm, a.stream,
                     static_cast<const uint16_t*>(FEAT ? f->k_raw : a.k), a.alpha,
                     FEAT ? f->beta_logit : a.beta, a.L, nc, Tfrag, Gws,
                     static_cast<const uint16_t*>(FEAT ? f->q_raw : nullptr),
                     static_cast<uint16_t*>(FEAT ? f->q_hat : nullptr),
                     static_cast<uint16_t*>(FEAT ? f->k_hat : nullptr), FEAT ? f->beta : nullptr,
                     XOUT ? *a.bwd_out : BwdFwdOut{});
  e = hipGetLastError();
  if (!a.bwd_out) prof_mark(kSlotChunkPrep, true, a.stream);
  return e;
}

template <int C, int DK>
hipError_t launch_c(const ChunkArgs& a) {
  const int nc = cdiv(a.L, C);
  uint4* Tfrag = static_cast<uint4*>(a.workspace);
  // The gated form's log-decay table follows the T fragments.
  float* Gws = reinterpret_cast<float*>(Tfrag + (size_t)a.B * a.H * nc * Frag<C>::chunk_u4);
  if (nc > 0) {
    hipError_t e;
    if constexpr (C == 128) {
      if (a.bwd_out) {
        e = launch_g<C, DK, false, false, true>(a, Tfrag, Gws);
        if (e != hipSuccess) return e;
        return launch_scan_mfma(a, Tfrag, nullptr);
      }
    }
    e = a.feat ? (a.alpha ? launch_g<C, DK, true, true>(a, Tfrag, Gws)
                          : launch_g<C, DK, false, true>(a, Tfrag, Gws))
               : (a.alpha ? launch_g<C, DK, true, false>(a, Tfrag, Gws)
                          : launch_g<C, DK, false, false>(a, Tfrag, Gws));
    if (e != hipSuccess) return e;
  }
  return launch_scan_mfma(a, Tfrag, a.alpha ? Gws : nullptr);
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
