// dn_scan_mfma.hip -- inter-chunk state scan and chunk outputs for bf16
// inputs on gfx950 matrix cores.
//
// The chunked form (page "GPT-2 から Kimi K3 まで、AI モデルの進化を解説",
// section "DeltaNet (Parallelizing linear transformers with delta rule)":
// every chunk's outputs follow from the previous chunk's final state and the
// chunk's own q, k, v).  For a chunk with rows K, Q, V, entering state S and
// T = (I + tril(diag(beta) K K^T, -1))^{-1} diag(beta) from the WY-prep kernel:
//     R     = V - K S
//     Delta = T R                 (the chunk's deltas, all at once)
//     S'    = S + K^T Delta
//     O     = Q S + tril(Q K^T) Delta   (diagonal included)
// The output is formed per 32-row sub-block b of the chunk from the state
// reached at the start of that sub-block, S_b = S + K_{<b}^T Delta_{<b}:
//     O_b = Q_b S_b + tril(Q_b K_b^T) Delta_b,
// which is the same sum regrouped (the strictly-lower blocks of tril(Q K^T)
// Delta are folded into S_b).  The S_b are exactly the partial sums of the
// state update, so only the 32 x 32 diagonal blocks of Q K^T are formed.
//
// Work split.  One 8-wave workgroup per (head, 16-column slice of d_v): the
// columns of S evolve independently, so each slice is its own scan and the
// slice's fp32 state stays in MFMA accumulators for the whole sequence.
// Workgroups are handed to the 8 XCDs round-robin by flat id; all slices of a
// head get the same flat id mod 8, so they run on one XCD and its L2 serves
// their shared k, q and T reads.
//   waves 0-3 ("chain"): the sequential part -- R, Delta, the state update --
//             at raised priority; each owns C/64 row tiles and d_k/64 state
//             tiles.
//   waves 4.. ("output"): one per sub-block; chunk c's outputs, including
//             its diagonal blocks of Q K^T, are formed during the next
//             chunk's R phase.
// Three barriers per chunk: R | Delta | state update.
//
// LDS: the chunk's K tile (double buffered; 16-byte chunks XOR-swizzled per
// row so that row reads and the transposing reads of K^T are free of bank
// conflicts), a ring of state snapshots S_b, R and Delta (Delta double
// buffered).  The snapshots, R and Delta are stored as split-bf16 operand
// planes (hi = bf16(x), lo = bf16(x - hi)); q and k are exact in bf16, so
// every product keeps roughly fp32 accuracy.
// A ragged last chunk loads clamped rows and zeroes them at first use
// (k, v rows and beta = 0 make those rows of R, Delta and T zero: no-ops);
// outputs past L are not stored.

#include "dn_common.h"
#include "dn_launch.h"
#include "dn_mfma.h"
#include "dn_tfrag.h"

namespace dn {
namespace scan {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

template <int C, int DK, int DV>
struct Cfg {
  static constexpr int NRT = C / 16;   // 16-row tiles of a chunk
  static constexpr int NSB = C / 32;   // 32-row sub-blocks of a chunk
  static constexpr int NKB = DK / 32;  // 32-wide blocks of d_k
  static constexpr int NCT = DV / 16;  // 16-column slices of d_v
  static constexpr int NCW = 4;        // chain waves
  static constexpr int NTHR = 512;     // 8 waves
  static constexpr int RPW = NRT / NCW;       // row tiles per chain wave
  static constexpr int DPW = DK / 16 / NCW;   // state tiles per chain wave
  static constexpr int NSLOT = NSB + 1;       // snapshot ring
  static constexpr int SPT = C * DK / (8 * NTHR);  // staged 16-byte k pieces per thread
  static constexpr int KELEMS = C * DK;       // one K buffer (bf16 elements)
  static constexpr int SPLANE = DK * 16;      // one plane of a state snapshot
  static constexpr int RPLANE = C * 16;       // one plane of R or Delta
  static constexpr int OFF_K = 0;
  static constexpr int OFF_SNAP = OFF_K + 2 * KELEMS;
  static constexpr int OFF_R = OFF_SNAP + NSLOT * 2 * SPLANE;
  static constexpr int OFF_D = OFF_R + 2 * RPLANE;
  static constexpr int TOTAL = OFF_D + 2 * 2 * RPLANE;
  static constexpr size_t bytes = (size_t)TOTAL * sizeof(uint16_t);
  static_assert(RPW >= 1 && DPW >= 1 && SPT >= 1, "shape");
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

// XOR swizzle of the 16-byte chunks of K-tile row `row` (conflict-free for
// 16-lane row reads and for the transposing 8-byte reads used for K^T).
template <int DK>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (DK == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return ((row >> 2) & 3) | ((row & 2) << 1);
}
// Element offset of 16-byte chunk `ch` (elements 8 ch .. 8 ch + 7) of row `row`.
template <int DK>
__device__ __forceinline__ int koff(int row, int ch) {
  return row * DK + ((ch ^ kswz<DK>(row)) << 3);
}

// Operand planes of a [rows x 16] split matrix: element (x, j) at
// ((x / 8) * 16 + j) * 8 + x % 8.
// B operand (contraction rows 32 blk + 8 g .. + 7, column j): 16 bytes here.
__device__ __forceinline__ int fo_b(int blk, int g, int j) { return ((4 * blk + g) * 16 + j) * 8; }
// D tile t of an MFMA (rows 16 t + 4 g .. + 3, column j): 8 bytes here.
__device__ __forceinline__ int fo_d(int t, int g, int j) {
  return ((2 * t + (g >> 1)) * 16 + j) * 8 + 4 * (g & 1);
}

__device__ __forceinline__ bf16x8 lds16(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ uint2 lds8(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }

// Transposing 8-byte LDS read: lane 4a + b of each 16-lane group receives
// element b of the 4 elements addressed by lanes a, a + 4, a + 8, a + 12.
__device__ __forceinline__ uint2 lds_tr(const uint16_t* p) {
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
  return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ void put_split(uint16_t* base, int plane, int off, f32x4 x) {
  uint2 hi, lo;
  split4(x, hi, lo);
  *reinterpret_cast<uint2*>(base + off) = hi;
  *reinterpret_cast<uint2*>(base + plane + off) = lo;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

template <int C, int DK, int DV, typename OT>
__global__ __launch_bounds__(512) void scan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ S0, OT* __restrict__ o,
    float* __restrict__ S_final, const uint4* __restrict__ Tfrag, int L, int nc, int BH) {
  using CF = Cfg<C, DK, DV>;
  constexpr int NRT = CF::NRT, NSB = CF::NSB, NKB = CF::NKB, NCT = CF::NCT;
  constexpr int RPW = CF::RPW, DPW = CF::DPW, SPT = CF::SPT, NSLOT = CF::NSLOT;
  constexpr int SPLANE = CF::SPLANE, RPLANE = CF::RPLANE, KELEMS = CF::KELEMS;
  constexpr int TB0 = 2;        // T blocks of a chain wave's first row tile (tiles 0..3)
  constexpr int TB1 = NRT / 2;  // ... of its second row tile (tiles NRT-4 .. NRT-1)

  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint16_t* const lds = reinterpret_cast<uint16_t*>(smem_raw);
  uint16_t* const Kbuf = lds + CF::OFF_K;
  uint16_t* const Snap = lds + CF::OFF_SNAP;
  uint16_t* const Rb = lds + CF::OFF_R;
  uint16_t* const Db = lds + CF::OFF_D;

  const int flat = blockIdx.x, xcd = flat & 7, sl = flat >> 3;
  const int ct = sl % NCT, bh = (sl / NCT) * 8 + xcd;
  if (bh >= BH) return;
  const int j0 = ct * 16;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, i16 = lane & 15;
  const bool chain = w < CF::NCW;
  const int a = w - CF::NCW;  // output wave index = sub-block
  const bool outw = !chain && a < NSB;

  const size_t sbase = (size_t)bh * DK * DV;
  const size_t tokh = (size_t)bh * L;
  const int rt0 = w, rt1 = NRT - 1 - w;  // chain row tiles (rt1 only if RPW == 2)

  // ---- chain state -------------------------------------------------------
  f32x4 sa[DPW], sb[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) { sa[i] = zero4(); sb[i] = zero4(); }
  uint32_t vreg[RPW][4];
  // One register array serves both roles (a wave is either a chain wave or
  // an output wave, so the compiler must not keep both sets live):
  //   chain waves:  the chunk's T fragments for the wave's row tiles;
  //   output waves: the q rows of the chunk whose outputs are due.
  constexpr int NTREG = 2 * TB0 + (RPW == 2 ? 2 * TB1 : 0);
  constexpr int NBANK = NTREG > 2 * NKB ? NTREG : 2 * NKB;
  uint4 bank[NBANK];
  uint4* const t0h = bank;
  uint4* const t0l = bank + TB0;
  uint4* const t1h = bank + 2 * TB0;
  uint4* const t1l = bank + 2 * TB0 + TB1;
  auto qreg = [&](int h, int kb) -> uint4& { return bank[h * NKB + kb]; };
  // ---- staging of the next chunk's k tile (all threads) ------------------
  uint4 kst[SPT];

  if (nc == 0) {
    if (chain && S_final) {
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        const int dt = DPW * w + i;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const size_t idx = sbase + (size_t)(16 * dt + 4 * g + r) * DV + j0 + i16;
          S_final[idx] = S0 ? S0[idx] : 0.f;
        }
      }
    }
    return;
  }

  auto valid_of = [&](int cc) { return min(C, L - cc * C); };
  auto slot_of = [&](int n) { return n % NSLOT; };

  auto stage_load = [&](int cc) {
    const int valid = valid_of(cc);
    const size_t t0 = tokh + (size_t)cc * C;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int e = i * CF::NTHR + tid, row = e / (DK / 8), ch = e % (DK / 8);
      kst[i] = *reinterpret_cast<const uint4*>(k + (t0 + min(row, valid - 1)) * DK + ch * 8);
    }
  };
  auto stage_store = [&](int cc, uint16_t* dst) {
    const int valid = valid_of(cc);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int e = i * CF::NTHR + tid, row = e / (DK / 8), ch = e % (DK / 8);
      const uint32_t m = row < valid ? 0xffffffffu : 0u;
      *reinterpret_cast<uint4*>(dst + koff<DK>(row, ch)) =
          make_uint4(kst[i].x & m, kst[i].y & m, kst[i].z & m, kst[i].w & m);
    }
  };
  auto v_load = [&](int cc) {
    const int valid = valid_of(cc);
    const size_t t0 = tokh + (size_t)cc * C;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int rt = i == 0 ? rt0 : rt1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rt + 4 * g + r;
        vreg[i][r] = v[(t0 + min(row, valid - 1)) * DV + j0 + i16];
      }
    }
  };
  auto t_load = [&](int cc) {
    const uint4* tb = Tfrag + ((size_t)bh * nc + cc) * Frag<C>::chunk_u4;
    const uint4* p0 = tb + (size_t)Frag<C>::base(rt0) * 128 + lane;
#pragma unroll
    for (int cb = 0; cb < TB0; ++cb) {
      if (cb <= rt0 / 2) {
        t0h[cb] = p0[(2 * cb) * 64];
        t0l[cb] = p0[(2 * cb + 1) * 64];
      }
    }
    if constexpr (RPW == 2) {
      const uint4* p1 = tb + (size_t)Frag<C>::base(rt1) * 128 + lane;
#pragma unroll
      for (int cb = 0; cb < TB1; ++cb) {
        if (cb <= rt1 / 2) {
          t1h[cb] = p1[(2 * cb) * 64];
          t1l[cb] = p1[(2 * cb + 1) * 64];
        }
      }
    }
  };
  auto q_load = [&](int cc) {
    const int valid = valid_of(cc);
    const size_t t0 = tokh + (size_t)cc * C;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = min(32 * a + 16 * h + i16, valid - 1);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        qreg(h, kb) = *reinterpret_cast<const uint4*>(q + (t0 + row) * DK + 32 * kb + 8 * g);
    }
  };

  // Outputs of chunk cc for sub-block a: Q_a S_a + tril(Q_a K_a^T) Delta_a,
  // with the q rows in qreg and chunk cc's k tile still in its LDS buffer.
  auto outputs = [&](int cc) {
    const int valid = valid_of(cc);
    const size_t t0 = tokh + (size_t)cc * C;
    const uint16_t* Kc = Kbuf + (cc & 1) * KELEMS;
    const uint16_t* Sn = Snap + slot_of(cc * NSB + a) * 2 * SPLANE;
    const uint16_t* Dc = Db + (cc & 1) * 2 * RPLANE;
    // Diagonal 32 x 32 block of Q K^T as transposed 16 x 16 tiles: lane
    // (i16, g) register r holds P[q = i16][k = 4 g + r] of its tile; the two
    // diagonal tiles keep k <= q, the tile above the diagonal is not needed.
    f32x4 p00 = zero4(), p01 = zero4(), p11 = zero4();
    f32x4 o0h = zero4(), o0l = zero4(), o1h = zero4(), o1l = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const bf16x8 K0 = lds16(Kc + koff<DK>(32 * a + i16, 4 * kb + g));
      const bf16x8 K1 = lds16(Kc + koff<DK>(32 * a + 16 + i16, 4 * kb + g));
      const bf16x8 Q0 = as_bf16x8(qreg(0, kb)), Q1 = as_bf16x8(qreg(1, kb));
      p00 = mfma16(K0, Q0, p00);
      p01 = mfma16(K0, Q1, p01);
      p11 = mfma16(K1, Q1, p11);
      const bf16x8 Sh = lds16(Sn + fo_b(kb, g, i16)), Sl = lds16(Sn + SPLANE + fo_b(kb, g, i16));
      o0h = mfma16(Q0, Sh, o0h);
      o0l = mfma16(Q0, Sl, o0l);
      o1h = mfma16(Q1, Sh, o1h);
      o1l = mfma16(Q1, Sl, o1l);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * g + r > i16) { p00[r] = 0.f; p11[r] = 0.f; }
    }
    // As A operands in the "d4" slot map: slots (g, 0..3) <-> k tile 2a rows
    // 4g..4g+3, slots (g, 4..7) <-> k tile 2a+1 rows 4g..4g+3.
    uint2 h00, l00, h01, l01, h11, l11;
    split4(p00, h00, l00);
    split4(p01, h01, l01);
    split4(p11, h11, l11);
    const uint4 ph0 = make_uint4(h00.x, h00.y, 0u, 0u), pl0 = make_uint4(l00.x, l00.y, 0u, 0u);
    const uint4 ph1 = make_uint4(h01.x, h01.y, h11.x, h11.y);
    const uint4 pl1 = make_uint4(l01.x, l01.y, l11.x, l11.y);
    const bf16x8 Dh = as_bf16x8(lds8(Dc + fo_d(2 * a, g, i16)), lds8(Dc + fo_d(2 * a + 1, g, i16)));
    const bf16x8 Dl = as_bf16x8(lds8(Dc + RPLANE + fo_d(2 * a, g, i16)),
                                lds8(Dc + RPLANE + fo_d(2 * a + 1, g, i16)));
    f32x4 x0 = mfma16(as_bf16x8(ph0), Dh, zero4());
    f32x4 x1 = mfma16(as_bf16x8(ph1), Dh, zero4());
    x0 = mfma16(as_bf16x8(ph0), Dl, x0);
    x1 = mfma16(as_bf16x8(ph1), Dl, x1);
    x0 = mfma16(as_bf16x8(pl0), Dh, x0);
    x1 = mfma16(as_bf16x8(pl1), Dh, x1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row0 = 32 * a + 4 * g + r, row1 = row0 + 16;
      if (row0 < valid) o[(t0 + row0) * DV + j0 + i16] = from_f32<OT>(o0h[r] + o0l[r] + x0[r]);
      if (row1 < valid) o[(t0 + row1) * DV + j0 + i16] = from_f32<OT>(o1h[r] + o1l[r] + x1[r]);
    }
  };

  // ---- prologue ------------------------------------------------------------
  if (chain) {
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int dt = DPW * w + i;
      if (S0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sa[i][r] = S0[sbase + (size_t)(16 * dt + 4 * g + r) * DV + j0 + i16];
      }
      put_split(Snap, SPLANE, fo_d(dt, g, i16), sa[i]);
    }
    v_load(0);
    t_load(0);
  }
  stage_load(0);
  stage_store(0, Kbuf);
  __syncthreads();

  for (int c = 0; c < nc; ++c) {
    const bool more = c + 1 < nc;
    const int valid = valid_of(c);
    const uint16_t* Kc = Kbuf + (c & 1) * KELEMS;
    uint16_t* Dc = Db + (c & 1) * 2 * RPLANE;

    // ---- phase A: R = V - K S (chain); outputs of chunk c-1 (output waves)
    if (more) stage_load(c + 1);
    if (chain) {
      const uint16_t* Sc = Snap + slot_of(c * NSB) * 2 * SPLANE;
      f32x4 rh[RPW], rl[RPW];
#pragma unroll
      for (int i = 0; i < RPW; ++i) { rh[i] = zero4(); rl[i] = zero4(); }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 Sh = lds16(Sc + fo_b(kb, g, i16)), Sl = lds16(Sc + SPLANE + fo_b(kb, g, i16));
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          const int rt = i == 0 ? rt0 : rt1;
          const bf16x8 Ka = lds16(Kc + koff<DK>(16 * rt + i16, 4 * kb + g));
          rh[i] = mfma16(Ka, Sh, rh[i]);
          rl[i] = mfma16(Ka, Sl, rl[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int rt = i == 0 ? rt0 : rt1;
        f32x4 R;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float vv = (16 * rt + 4 * g + r) < valid ? bf16_to_f32(vreg[i][r]) : 0.f;
          R[r] = vv - (rh[i][r] + rl[i][r]);
        }
        put_split(Rb, RPLANE, fo_d(rt, g, i16), R);
      }
    } else if (outw) {
      if (c > 0) outputs(c - 1);
      q_load(c);
    }
    __syncthreads();

    // ---- phase B: Delta = T R (chain) ---------------------------------------
    if (chain) {
      if (more) v_load(c + 1);
      {
        f32x4 d0 = zero4(), d1 = zero4(), d2 = zero4();
#pragma unroll
        for (int cb = 0; cb < TB0; ++cb) {
          if (cb <= rt0 / 2) {
            const bf16x8 Rh = lds16(Rb + fo_b(cb, g, i16)), Rl = lds16(Rb + RPLANE + fo_b(cb, g, i16));
            d0 = mfma16(as_bf16x8(t0h[cb]), Rh, d0);
            d1 = mfma16(as_bf16x8(t0h[cb]), Rl, d1);
            d2 = mfma16(as_bf16x8(t0l[cb]), Rh, d2);
          }
        }
        put_split(Dc, RPLANE, fo_d(rt0, g, i16), d0 + d1 + d2);
      }
      if constexpr (RPW == 2) {
        f32x4 d0 = zero4(), d1 = zero4(), d2 = zero4();
#pragma unroll
        for (int cb = 0; cb < TB1; ++cb) {
          if (cb <= rt1 / 2) {
            const bf16x8 Rh = lds16(Rb + fo_b(cb, g, i16)), Rl = lds16(Rb + RPLANE + fo_b(cb, g, i16));
            d0 = mfma16(as_bf16x8(t1h[cb]), Rh, d0);
            d1 = mfma16(as_bf16x8(t1h[cb]), Rl, d1);
            d2 = mfma16(as_bf16x8(t1l[cb]), Rh, d2);
          }
        }
        put_split(Dc, RPLANE, fo_d(rt1, g, i16), d0 + d1 + d2);
      }
    }
    __syncthreads();

    // ---- phase C: S += K^T Delta with sub-block snapshots (chain);
    //      stage k of chunk c+1 (all waves).
    if (chain) {
      if (more) t_load(c + 1);
      const int m = i16 >> 2, ap = i16 & 3;
#pragma unroll
      for (int b = 0; b < NSB; ++b) {
        const bf16x8 Dh = lds16(Dc + fo_b(b, g, i16)), Dl = lds16(Dc + RPLANE + fo_b(b, g, i16));
        const int row = 32 * b + 8 * g + m;
#pragma unroll
        for (int i = 0; i < DPW; ++i) {
          const int dt = DPW * w + i;
          const int ch = 2 * dt + (ap >> 1), sub = 4 * (ap & 1);
          const uint2 lo4 = lds_tr(Kc + koff<DK>(row, ch) + sub);
          const uint2 hi4 = lds_tr(Kc + koff<DK>(row + 4, ch) + sub);
          const bf16x8 A = as_bf16x8(lo4, hi4);
          sa[i] = mfma16(A, Dh, sa[i]);
          sb[i] = mfma16(A, Dl, sb[i]);
        }
        uint16_t* dst = Snap + slot_of(c * NSB + b + 1) * 2 * SPLANE;
#pragma unroll
        for (int i = 0; i < DPW; ++i) put_split(dst, SPLANE, fo_d(DPW * w + i, g, i16), sa[i] + sb[i]);
      }
#pragma unroll
      for (int i = 0; i < DPW; ++i) { sa[i] = sa[i] + sb[i]; sb[i] = zero4(); }
    }
    if (more) stage_store(c + 1, Kbuf + ((c + 1) & 1) * KELEMS);
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------
  if (outw) outputs(nc - 1);
  if (chain && S_final) {
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int dt = DPW * w + i;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S_final[sbase + (size_t)(16 * dt + 4 * g + r) * DV + j0 + i16] = sa[i][r];
    }
  }
}

template <int C, int DK, int DV, typename OT>
hipError_t launch_t(const ChunkArgs& a, const uint4* Tfrag) {
  using CF = Cfg<C, DK, DV>;
  const int nc = cdiv(a.L, C);
  const int BH = a.B * a.H;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_kernel<C, DK, DV, OT>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)CF::bytes);
  if (e != hipSuccess) return e;
  const int groups = cdiv(BH, 8) * 8 * CF::NCT;
  prof_mark(kSlotChunkScan, false, a.stream);
  hipLaunchKernelGGL((scan_kernel<C, DK, DV, OT>), dim3(groups), dim3(CF::NTHR), CF::bytes,
                     a.stream, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), a.S0,
                     static_cast<OT*>(a.o), a.S_final, Tfrag, a.L, nc, BH);
  e = hipGetLastError();
  prof_mark(kSlotChunkScan, true, a.stream);
  return e;
}

template <int C, int DK, int DV>
hipError_t launch_o(const ChunkArgs& a, const uint4* Tfrag) {
  return a.out_dtype == 0 ? launch_t<C, DK, DV, float>(a, Tfrag)
                          : launch_t<C, DK, DV, bf16>(a, Tfrag);
}

template <int C>
hipError_t launch_c(const ChunkArgs& a, const uint4* Tfrag) {
  if (a.d_k == 64 && a.d_v == 64) return launch_o<C, 64, 64>(a, Tfrag);
  if (a.d_k == 64 && a.d_v == 128) return launch_o<C, 64, 128>(a, Tfrag);
  if (a.d_k == 128 && a.d_v == 64) return launch_o<C, 128, 64>(a, Tfrag);
  return launch_o<C, 128, 128>(a, Tfrag);
}

}  // namespace scan

hipError_t launch_scan_mfma(const ChunkArgs& a, const uint4* Tfrag) {
  return a.C == 64 ? scan::launch_c<64>(a, Tfrag) : scan::launch_c<128>(a, Tfrag);
}

}  // namespace dn
