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
// conflicts), the state snapshots, R and Delta (Delta double buffered).  The
// entering state, R and Delta are stored as split-bf16 operand planes
// (hi = bf16(x), lo = bf16(x - hi)); the states inside a chunk are stored as
// fp32 (in 4-row groups, see fo_f) and split by their reader.  q and k are
// exact in bf16, so every product keeps roughly fp32 accuracy.
// Global reads go through buffer descriptors made per chunk (base address in
// scalar registers, a fixed byte offset per lane), so a chunk step spends no
// vector instructions on addresses, and the descriptor's range check returns
// zero for rows past L: a ragged last chunk reads k and v rows of zero (with
// beta = 0 those rows of R, Delta and T are zero: no-ops); outputs past L
// are not stored.
//
// Each split product accumulates all of its passes (hi*hi, hi*lo, lo*hi) in
// one fp32 accumulator, and the outputs are formed as transposed tiles,
// (Q S + P Delta)^T = S^T Q^T + Delta^T P^T: the same operand registers with
// A and B swapped, which leaves each lane holding 4 consecutive columns of
// one output row, stored to HBM as one 16-byte write.
//
// Gated form (GATED; Gated DeltaNet, article "How a Baseten Engineer Traced 7
// Years of Attention Mechanism Evolution", Gated DeltaNet section: the state
// is decayed by alpha_t before each precise write).  With the chunk's
// cumulative log-decays g_r (from the prep kernel; every factor below has a
// non-positive exponent) and G_b = g of the last row before sub-block b
// (G_0 = 0):
//     R       = V - diag(e^g) K S
//     S_{b+1} = e^{G_{b+1} - G_b} S_b + K_b^T diag(e^{G_{b+1} - g}) Delta_b
//     O_b     = diag(e^{g - G_b}) Q_b S_b + (tril(Q_b K_b^T) o e^{g_r - g_i}) Delta_b
// The chain waves write a second, decayed copy of Delta for the state update;
// the output waves decay their rows and their diagonal Q K^T block.  The
// per-row factors e^{g_r}, e^{G_{b+1} - g_r} and e^{g_r - G_b} are computed
// once per chunk by the output waves while they stage the chunk, and kept in
// LDS next to g, so the chain waves only multiply.

#include "dn_buffer.h"
#include "dn_common.h"
#include "dn_launch.h"
#include "dn_mfma.h"
#include "dn_ktile.h"
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
  // State snapshots: the state entering a chunk, S_c, as split planes in a
  // 2-slot ring (slot c & 1); the states inside the chunk, S_{c,b} for
  // b = 1 .. NSB-1, as plain fp32 (split by the output waves that read them).
  static constexpr int NFSNAP = NSB - 1;
  static constexpr int SPT = C * DK / (8 * NTHR);  // staged 16-byte k pieces per thread
  static constexpr int KELEMS = C * DK;       // one K buffer (bf16 elements)
  static constexpr int SPLANE = DK * 16;      // one plane of a state snapshot
  static constexpr int RPLANE = C * 16;       // one plane of R or Delta
  static constexpr int OFF_K = 0;
  static constexpr int OFF_SNAP = OFF_K + 2 * KELEMS;          // [2][hi, lo planes]
  static constexpr int OFF_FSNAP = OFF_SNAP + 2 * 2 * SPLANE;   // [NFSNAP][DK*16 fp32]
  static constexpr int OFF_R = OFF_FSNAP + NFSNAP * 2 * SPLANE;
  static constexpr int OFF_D = OFF_R + 2 * RPLANE;
  static constexpr int OFF_V = OFF_D + 2 * 2 * RPLANE;   // [2][C][16] bf16 v slice
  static constexpr int OFF_DT = OFF_V + 2 * C * 16;       // decayed Delta planes (gated form)
  // Gated form: per slot (chunk parity), 4 rows of C fp32: g, e^{g},
  // e^{G_{b+1} - g}, e^{g - G_b} (b = the row's sub-block).
  static constexpr int OFF_G = OFF_DT + 2 * RPLANE;
  static constexpr int TOTAL = OFF_G + 2 * 4 * C * 2;
  static constexpr size_t bytes = (size_t)TOTAL * sizeof(uint16_t);
  static_assert(RPW >= 1 && DPW >= 1 && SPT >= 1, "shape");
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Operand planes of a [rows x 16] split matrix: element (x, j) at
// ((x / 8) * 16 + j) * 8 + x % 8.
// B operand (contraction rows 32 blk + 8 g .. + 7, column j): 16 bytes here.
__device__ __forceinline__ int fo_b(int blk, int g, int j) { return ((4 * blk + g) * 16 + j) * 8; }
// D tile t of an MFMA (rows 16 t + 4 g .. + 3, column j): 8 bytes here.
__device__ __forceinline__ int fo_d(int t, int g, int j) {
  return ((2 * t + (g >> 1)) * 16 + j) * 8 + 4 * (g & 1);
}

// fp32 state snapshot [DK x 16]: the 4-row group q (rows 4 q .. 4 q + 3) of
// column j as 16 contiguous bytes at float offset (q * 16 + j) * 4, so that a
// 16-lane group reading or writing one 4-row group touches 256 contiguous
// bytes (no LDS bank conflict).
__device__ __forceinline__ int fo_f(int q, int j) { return (q * 16 + j) * 4; }

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

// BWD: the forward pass of the backward (128-token chunks here, 64-token
// blocks there).  Instead of o, the kernel writes for every 64-token block of
// the backward's workspace the state entering it, R = V - K S from that
// state, and Delta (the deltas do not depend on the chunking):
//   - the chain waves store the entering state of the chunk and, after the
//     state update's second sub-block, that of the second block; R of the
//     first block (rows of R = V - K S_c); Delta of both blocks;
//   - the output waves of sub-blocks 2 and 3 form R of the second block,
//     V - K S_{c,2} with S_{c,2} the state after 64 rows, in the next
//     chunk's R phase, as they form outputs otherwise (q is not read).
template <int C, int DK, int DV, typename OT, bool GATED, bool BWD = false>
__global__ __launch_bounds__(512) void scan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ S0, OT* __restrict__ o,
    float* __restrict__ S_final, const uint4* __restrict__ Tfrag, const float* __restrict__ Gws,
    int L, int nc, int BH, BwdFwdOut bo) {
  static_assert(!BWD || (C == 128 && !GATED), "the backward's forward pass: plain form, C = 128");
  using CF = Cfg<C, DK, DV>;
  constexpr int NRT = CF::NRT, NSB = CF::NSB, NKB = CF::NKB, NCT = CF::NCT;
  constexpr int RPW = CF::RPW, DPW = CF::DPW, SPT = CF::SPT;
  constexpr int SPLANE = CF::SPLANE, RPLANE = CF::RPLANE, KELEMS = CF::KELEMS;
  constexpr int TB0 = 2;        // T blocks of a chain wave's first row tile (tiles 0..3) at most
  constexpr int TB1 = NRT / 2;  // ... of its second row tile (tiles NRT-4 .. NRT-1)
  // Register slots for one chunk's T blocks of a chain wave: row tile rt0's
  // block cb in slot cb, row tile rt1's block cb in slot NTS - 1 - cb.  The
  // two tiles of a wave have NRT/2 + 1 blocks together, so every slot is
  // loaded once and used once, and the indices stay compile-time constants.
  constexpr int NTS = RPW == 2 ? NRT / 2 + 1 : TB0;

  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint16_t* const lds = reinterpret_cast<uint16_t*>(smem_raw);
  uint16_t* const Kbuf = lds + CF::OFF_K;
  uint16_t* const Snap = lds + CF::OFF_SNAP;
  float* const Fsnap = reinterpret_cast<float*>(lds + CF::OFF_FSNAP);
  uint16_t* const Rb = lds + CF::OFF_R;
  uint16_t* const Db = lds + CF::OFF_D;
  uint16_t* const Vbuf = lds + CF::OFF_V;
  uint16_t* const DTb = lds + CF::OFF_DT;
  float* const Gs = reinterpret_cast<float*>(lds + CF::OFF_G);

  const int flat = blockIdx.x, xcd = flat & 7, sl = flat >> 3;
  const int ct = sl % NCT, bh = (sl / NCT) * 8 + xcd;
  if (bh >= BH) return;
  const int j0 = ct * 16;
  // (The wave index is the same in every lane: read from the first lane it
  // lives in a scalar register, and so does everything derived from it.)
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, i16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool chain = w < CF::NCW;
  const size_t sbase = (size_t)bh * DK * DV;
  const size_t tokh = (size_t)bh * L;
  // BWD: 64-token block nb of this head in the backward's workspace.
  auto bblk = [&](int nb) { return bo.ws + ((size_t)bh * bo.nb + nb) * bo.block; };

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
  // Descriptors over chunk cc's rows of q, k (d_k wide) and v (d_v wide): rows
  // past L read as zero.
  auto rows_rsrc = [&](const uint16_t* base, int width, int cc) {
    const size_t t0 = tokh + (size_t)cc * C;
    return make_rsrc(base + t0 * width, (uint32_t)valid_of(cc) * width * 2);
  };

  // Staging of a chunk's k tile into LDS, shared by all 512 threads.  The
  // global loads of the next chunk are issued early and consumed by the
  // store one or two phases later.
  uint4 kst[SPT];
  uint32_t kvoff[SPT];
  int kdst[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int e = i * CF::NTHR + tid, row = e / (DK / 8), ch = e % (DK / 8);
    kvoff[i] = (uint32_t)(row * DK + ch * 8) * 2;
    kdst[i] = koff<DK>(row, ch);
  }
  auto stage_load = [&](int cc) {
    const rsrc_t rk = rows_rsrc(k, DK, cc);
#pragma unroll
    for (int i = 0; i < SPT; ++i) kst[i] = bload16(rk, kvoff[i], 0);
  };
  auto stage_store = [&](uint16_t* dst) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) *reinterpret_cast<uint4*>(dst + kdst[i]) = kst[i];
  };

  // Each role runs its own loop with the same three barriers per chunk, and
  // every global load inside a loop is unconditional (the chunk index is
  // clamped on the last step), so the compiler's wait counts stay exact and
  // the loads of the next chunk remain in flight across phases.
  if (chain) {
    // ======================= chain waves =====================================
    __builtin_amdgcn_s_setprio(2);
    const int rt0 = w, rt1 = NRT - 1 - w;  // row tiles (rt1 only if RPW == 2)
    f32x4 st[DPW];
    // T fragments of one chunk for this wave's row tiles, loaded at the very
    // start of the chunk's step (ahead of every other wave's loads of that
    // step) and used in its Delta phase.
    struct TRegs {
      uint4 h[NTS], l[NTS];
    };
    TRegs tA;
    // Byte offset of slot sl's block within a chunk's fragments (wave-uniform).
    int tsoff[NTS];
#pragma unroll
    for (int sl = 0; sl < NTS; ++sl) {
      // (RPW == 1: a slot past the tile's last block re-reads block 0, unused.)
      const bool first = RPW == 1 || sl <= rt0 / 2;
      const int blk = RPW == 1 ? (sl <= rt0 / 2 ? sl : 0) : (first ? sl : NTS - 1 - sl);
      tsoff[sl] = (Frag<C>::base(first ? rt0 : rt1) + blk) * 128 * 16;
    }
    auto t_load = [&](int cc, TRegs& t) {
      const rsrc_t rt = make_rsrc(Tfrag + ((size_t)bh * nc + cc) * Frag<C>::chunk_u4,
                                  (uint32_t)(Frag<C>::chunk_u4 * 16));
#pragma unroll
      for (int sl = 0; sl < NTS; ++sl) {
        t.h[sl] = bload16(rt, lane * 16, tsoff[sl]);
        t.l[sl] = bload16(rt, lane * 16, tsoff[sl] + 64 * 16);
      }
    };

#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int dt = DPW * w + i;
      st[i] = zero4();
      if (S0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          st[i][r] = S0[sbase + (size_t)(16 * dt + 4 * g + r) * DV + j0 + i16];
      }
      put_split(Snap, SPLANE, fo_d(dt, g, i16), st[i]);
    }
    stage_load(0);
    stage_store(Kbuf);
    __syncthreads();

    const int m = i16 >> 2, ap = i16 & 3;
    // Gated form: Delta rows 16 rt + 4 g + r of chunk c scaled by
    // e^{G_{b+1} - g_row}, G_{b+1} = g of the last row of the row's sub-block.
    auto decay_rows = [&](int rt, f32x4 x, int c) {
      const f32x4 f = *reinterpret_cast<const f32x4*>(Gs + (c & 1) * 4 * C + 2 * C + 16 * rt + 4 * g);
      return x * f;
    };
    // BWD: Delta rows 16 rt + 4 g + r of chunk c into block 2c or 2c + 1
    // (a block past the sequence's last is not written).
    auto store_delta = [&](int rt, f32x4 x, int c) {
      const int nb = 2 * c + rt / (NRT / 2);
      if (nb < bo.nb) {
        float* dd = bblk(nb) + bo.d;
#pragma unroll
        for (int r = 0; r < 4; ++r) dd[(size_t)(16 * (rt % (NRT / 2)) + 4 * g + r) * DV + j0 + i16] = x[r];
      }
    };
    auto step = [&](int c, TRegs& tc) {
      const int cn = min(c + 1, nc - 1);
      const uint16_t* Kc = Kbuf + (c & 1) * KELEMS;
      uint16_t* Dc = Db + (c & 1) * 2 * RPLANE;

      // ---- phase A: R = V - K S ----------------------------------------------
      t_load(c, tc);
      stage_load(cn);
      if constexpr (BWD) {  // the state entering block 2c
        float* sd = bblk(2 * c) + bo.s;
#pragma unroll
        for (int i = 0; i < DPW; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) sd[(size_t)(16 * (DPW * w + i) + 4 * g + r) * DV + j0 + i16] = st[i][r];
      }
      {
        const uint16_t* Sc = Snap + (c & 1) * 2 * SPLANE;
        // All LDS operands of the phase are read up front, then multiplied.
        bf16x8 Sh[NKB], Sl[NKB], Ka[RPW][NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          Sh[kb] = lds16(Sc + fo_b(kb, g, i16));
          Sl[kb] = lds16(Sc + SPLANE + fo_b(kb, g, i16));
#pragma unroll
          for (int i = 0; i < RPW; ++i)
            Ka[i][kb] = lds16(Kc + koff<DK>(16 * (i == 0 ? rt0 : rt1) + i16, 4 * kb + g));
        }
        f32x4 ks[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) ks[i] = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int i = 0; i < RPW; ++i) ks[i] = mfma_split2(Ka[i][kb], Sh[kb], Sl[kb], ks[i]);
        }
        // v in the D layout straight from the staged row-major slice: the
        // transposing read gives lane (i16, g) rows 16 rt + 4 g .. + 3 of
        // column i16 (rows past L were staged as zero).
        const uint16_t* Vc = Vbuf + (c & 1) * C * 16;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          const int rt = i == 0 ? rt0 : rt1;
          const uint2 vv = lds_tr(Vc + (16 * rt + 4 * g + m) * 16 + 4 * ap);
          const float v4[4] = {bf16_to_f32(vv.x & 0xffffu), bf16_to_f32(vv.x >> 16),
                               bf16_to_f32(vv.y & 0xffffu), bf16_to_f32(vv.y >> 16)};
          f32x4 R;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float kv = ks[i][r];
            if constexpr (GATED) kv *= Gs[(c & 1) * 4 * C + C + 16 * rt + 4 * g + r];
            R[r] = v4[r] - kv;
          }
          put_split(Rb, RPLANE, fo_d(rt, g, i16), R);
          if constexpr (BWD) {  // R of block 2c (rows 0..63, from the chunk's entering state)
            if (rt < NRT / 2) {
              float* rd = bblk(2 * c) + bo.r;
#pragma unroll
              for (int r = 0; r < 4; ++r) rd[(size_t)(16 * rt + 4 * g + r) * DV + j0 + i16] = R[r];
            }
          }
        }
      }
      __syncthreads();

      // ---- phase B: Delta = T R ------------------------------------------------
      {
        constexpr int NRB = RPW == 2 ? TB1 : TB0;  // R blocks any tile of this wave needs
        const int nrb = (RPW == 2 ? rt1 : rt0) / 2 + 1;
        bf16x8 Rh[NRB], Rl[NRB];
#pragma unroll
        for (int cb = 0; cb < NRB; ++cb) {
          if (cb < nrb) {  // d4 slot map, matching the T fragments
            Rh[cb] = as_bf16x8(lds8(Rb + fo_d(2 * cb, g, i16)), lds8(Rb + fo_d(2 * cb + 1, g, i16)));
            Rl[cb] = as_bf16x8(lds8(Rb + RPLANE + fo_d(2 * cb, g, i16)),
                               lds8(Rb + RPLANE + fo_d(2 * cb + 1, g, i16)));
          }
        }
        f32x4 d0 = zero4();
#pragma unroll
        for (int cb = 0; cb < TB0; ++cb) {
          if (cb <= rt0 / 2)
            d0 = mfma_split3(as_bf16x8(tc.h[cb]), as_bf16x8(tc.l[cb]), Rh[cb], Rl[cb], d0);
        }
        if constexpr (RPW == 2) {
          f32x4 e0 = zero4();
#pragma unroll
          for (int cb = 0; cb < TB1; ++cb) {
            if (cb <= rt1 / 2)
              e0 = mfma_split3(as_bf16x8(tc.h[NTS - 1 - cb]), as_bf16x8(tc.l[NTS - 1 - cb]), Rh[cb],
                               Rl[cb], e0);
          }
          put_split(Dc, RPLANE, fo_d(rt1, g, i16), e0);
          if constexpr (GATED) put_split(DTb, RPLANE, fo_d(rt1, g, i16), decay_rows(rt1, e0, c));
          if constexpr (BWD) store_delta(rt1, e0, c);
        }
        put_split(Dc, RPLANE, fo_d(rt0, g, i16), d0);
        if constexpr (BWD) store_delta(rt0, d0, c);
        if constexpr (GATED) put_split(DTb, RPLANE, fo_d(rt0, g, i16), decay_rows(rt0, d0, c));
      }
      __syncthreads();

      // ---- phase C: S += K^T Delta, snapshot after every sub-block -------------
      {
        bf16x8 Dh[NSB], Dl[NSB], Kt[NSB][DPW];
        const uint16_t* Du = GATED ? DTb : Dc;  // the state update takes the decayed copy
#pragma unroll
        for (int b = 0; b < NSB; ++b) {
          Dh[b] = lds16(Du + fo_b(b, g, i16));
          Dl[b] = lds16(Du + RPLANE + fo_b(b, g, i16));
          const int row = 32 * b + 8 * g + m;
#pragma unroll
          for (int i = 0; i < DPW; ++i) {
            const int ch = 2 * (DPW * w + i) + (ap >> 1), sub = 4 * (ap & 1);
            Kt[b][i] = as_bf16x8(lds_tr(Kc + koff<DK>(row, ch) + sub),
                                 lds_tr(Kc + koff<DK>(row + 4, ch) + sub));
          }
        }
#pragma unroll
        for (int b = 0; b < NSB; ++b) {
          if constexpr (GATED) {  // S_b -> e^{G_{b+1} - G_b} S_b  (= e^{g - G_b} at the block's last row)
            const float f = Gs[(c & 1) * 4 * C + 3 * C + 32 * b + 31];
#pragma unroll
            for (int i = 0; i < DPW; ++i) st[i] *= f;
          }
#pragma unroll
          for (int i = 0; i < DPW; ++i) st[i] = mfma_split2(Kt[b][i], Dh[b], Dl[b], st[i]);
          if (b + 1 < NSB) {
            float* dst = Fsnap + b * DK * 16;
#pragma unroll
            for (int i = 0; i < DPW; ++i)
              *reinterpret_cast<f32x4*>(dst + fo_f(4 * (DPW * w + i) + g, i16)) = st[i];
            if constexpr (BWD) {  // the state entering block 2c + 1
              if (b == NSB / 2 - 1 && 2 * c + 1 < bo.nb) {
                float* sd = bblk(2 * c + 1) + bo.s;
#pragma unroll
                for (int i = 0; i < DPW; ++i)
#pragma unroll
                  for (int r = 0; r < 4; ++r)
                    sd[(size_t)(16 * (DPW * w + i) + 4 * g + r) * DV + j0 + i16] = st[i][r];
              }
            }
          } else {
            uint16_t* dst = Snap + ((c + 1) & 1) * 2 * SPLANE;
#pragma unroll
            for (int i = 0; i < DPW; ++i) put_split(dst, SPLANE, fo_d(DPW * w + i, g, i16), st[i]);
          }
        }
      }
      stage_store(Kbuf + ((c + 1) & 1) * KELEMS);
      __syncthreads();
    };
    for (int c = 0; c < nc; ++c) step(c, tA);

    if (S_final) {
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        const int dt = DPW * w + i;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S_final[sbase + (size_t)(16 * dt + 4 * g + r) * DV + j0 + i16] = st[i][r];
      }
    }
  } else {
    // ======================= output waves ====================================
    // Wave 4 + a owns sub-block a (row tiles 2a, 2a+1).  With C = 64 only
    // waves 4 and 5 have a sub-block; the others load and stage like the rest
    // but skip the arithmetic.
    const int a = w - CF::NCW;
    const bool outw = a < NSB;
    const int aq = outw ? a : 0;
    uint4 qreg[2][NKB];
    uint32_t qvoff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) qvoff[h] = (uint32_t)((32 * aq + 16 * h + i16) * DK + 8 * g) * 2;
    // The chunk's 16-column v slice is staged row-major into LDS by the
    // output waves' 256 threads (16 bytes each: row tl / 2, half tl % 2);
    // rows past L read as zero.
    const int tl = tid - CF::NCW * 64;  // 0 .. 255
    const int vrow = min(tl >> 1, C - 1), vhalf = tl & 1;
    const uint32_t vvoff = (uint32_t)(vrow * DV + j0 + 8 * vhalf) * 2;
    // (Gated form: the chunk's C log-decays ride along, 16 bytes per thread,
    // into slot `gslot` of Gs, the parity of the chunk step that uses them.)
    uint4 vst;
    float4 gst;
    float gb0, gb1;  // G_b and G_{b+1} of the sub-block of this thread's 4 rows
    const int grow4 = 4 * (tl % (C / 4)), gblk = grow4 >> 5;
    auto v_stage_load = [&](int cc) {
      vst = bload16(rows_rsrc(v, DV, cc), vvoff, 0);
      if constexpr (GATED) {
        const float* gsrc = Gws + ((size_t)bh * nc + cc) * C;
        gst = *reinterpret_cast<const float4*>(gsrc + grow4);
        gb0 = gsrc[max(32 * gblk - 1, 0)];
        gb1 = gsrc[32 * gblk + 31];
      }
    };
    auto v_stage_store = [&](uint16_t* dst, int gslot) {
      if (tl < 2 * C) *reinterpret_cast<uint4*>(dst + vrow * 16 + 8 * vhalf) = vst;
      if constexpr (GATED) {
        if (tl < C / 4) {
          const float G0 = gblk > 0 ? gb0 : 0.f;
          const float gv[4] = {gst.x, gst.y, gst.z, gst.w};
          float* dst = Gs + gslot * 4 * C + grow4;
          *reinterpret_cast<float4*>(dst) = gst;
          *reinterpret_cast<float4*>(dst + C) =
              make_float4(__expf(gv[0]), __expf(gv[1]), __expf(gv[2]), __expf(gv[3]));
          *reinterpret_cast<float4*>(dst + 2 * C) =
              make_float4(__expf(gb1 - gv[0]), __expf(gb1 - gv[1]), __expf(gb1 - gv[2]), __expf(gb1 - gv[3]));
          *reinterpret_cast<float4*>(dst + 3 * C) =
              make_float4(__expf(gv[0] - G0), __expf(gv[1] - G0), __expf(gv[2] - G0), __expf(gv[3] - G0));
        }
      }
    };
    auto q_load = [&](int cc) {
      const rsrc_t rq = rows_rsrc(q, DK, cc);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) qreg[h][kb] = bload16(rq, qvoff[h] + 64 * kb, 0);
      }
    };
    // Diagonal 32 x 32 block of Q K^T of chunk cc for sub-block a, as split
    // operands of the P Delta product.  Computed as transposed 16 x 16
    // tiles: lane (i16, g) register r holds P[q = i16][k = 4 g + r] of its
    // tile; the two diagonal tiles keep k <= q, the tile above the diagonal is
    // not needed.  "d4" slot map: slots (g, 0..3) <-> k tile 2a rows
    // 4g..4g+3, slots (g, 4..7) <-> k tile 2a+1 rows 4g..4g+3.
    uint4 ph0, pl0, ph1, pl1;
    auto diag_qk = [&](int cc) {
      const uint16_t* Kc = Kbuf + (cc & 1) * KELEMS;
      bf16x8 K0[NKB], K1[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        K0[kb] = lds16(Kc + koff<DK>(32 * a + i16, 4 * kb + g));
        K1[kb] = lds16(Kc + koff<DK>(32 * a + 16 + i16, 4 * kb + g));
      }
      f32x4 p00 = zero4(), p01 = zero4(), p11 = zero4();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 Q0 = as_bf16x8(qreg[0][kb]), Q1 = as_bf16x8(qreg[1][kb]);
        p00 = mfma16(K0[kb], Q0, p00);
        p01 = mfma16(K0[kb], Q1, p01);
        p11 = mfma16(K1[kb], Q1, p11);
      }
      if constexpr (GATED) {  // P[q][k] e^{g_q - g_k}, k <= q
        const float* gc = Gs + (cc & 1) * 4 * C + 32 * a;
        const float gq0 = gc[i16], gq1 = gc[16 + i16];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gk0 = gc[4 * g + r], gk1 = gc[16 + 4 * g + r];
          p00[r] *= __expf(fminf(gq0 - gk0, 0.f));
          p01[r] *= __expf(fminf(gq1 - gk0, 0.f));
          p11[r] *= __expf(fminf(gq1 - gk1, 0.f));
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (4 * g + r > i16) { p00[r] = 0.f; p11[r] = 0.f; }
      }
      uint2 h00, l00, h01, l01, h11, l11;
      split4(p00, h00, l00);
      split4(p01, h01, l01);
      split4(p11, h11, l11);
      ph0 = make_uint4(h00.x, h00.y, 0u, 0u);
      pl0 = make_uint4(l00.x, l00.y, 0u, 0u);
      ph1 = make_uint4(h01.x, h01.y, h11.x, h11.y);
      pl1 = make_uint4(l01.x, l01.y, l11.x, l11.y);
    };
    // Outputs of chunk cc for sub-block a, (Q_a S_a + tril(Q_a K_a^T) Delta_a)^T
    // = S_a^T Q_a^T + Delta_a^T P^T, with chunk cc's q rows in qreg and its
    // diagonal Q K^T block in ph/pl: lane (i16, g) ends with row 32 a + 16 h +
    // i16 of o, columns 4 g .. 4 g + 3 of the slice.
    auto outputs = [&](int cc) {
      const int valid = valid_of(cc);
      const size_t t0 = tokh + (size_t)cc * C;
      const uint16_t* Dc = Db + (cc & 1) * 2 * RPLANE;
      bf16x8 Sh[NKB], Sl[NKB];
      if (a == 0) {
        const uint16_t* Sn = Snap + (cc & 1) * 2 * SPLANE;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          Sh[kb] = lds16(Sn + fo_b(kb, g, i16));
          Sl[kb] = lds16(Sn + SPLANE + fo_b(kb, g, i16));
        }
      } else {
        const float* Sn = Fsnap + (a - 1) * DK * 16;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          // rows 32 kb + 8 g .. + 7: the 4-row groups 8 kb + 2 g and 8 kb + 2 g + 1
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(Sn + fo_f(8 * kb + 2 * g, i16));
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(Sn + fo_f(8 * kb + 2 * g + 1, i16));
          uint2 h0, l0, h1, l1;
          split4(x0, h0, l0);
          split4(x1, h1, l1);
          Sh[kb] = as_bf16x8(h0, h1);
          Sl[kb] = as_bf16x8(l0, l1);
        }
      }
      const bf16x8 Dh = as_bf16x8(lds8(Dc + fo_d(2 * a, g, i16)), lds8(Dc + fo_d(2 * a + 1, g, i16)));
      const bf16x8 Dl = as_bf16x8(lds8(Dc + RPLANE + fo_d(2 * a, g, i16)),
                                  lds8(Dc + RPLANE + fo_d(2 * a + 1, g, i16)));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const bf16x8 Qh = as_bf16x8(qreg[h][kb]);
          acc = mfma16(Sh[kb], Qh, acc);
          acc = mfma16(Sl[kb], Qh, acc);
        }
        const int row = 32 * a + 16 * h + i16;
        if constexpr (GATED)  // row of Q_a S_a decayed by e^{g_row - G_a}
          acc *= Gs[(cc & 1) * 4 * C + 3 * C + row];
        acc = mfma_split3(Dh, Dl, as_bf16x8(h == 0 ? ph0 : ph1), as_bf16x8(h == 0 ? pl0 : pl1), acc);
        if (row < valid) {
          OT* dst = o + (t0 + row) * DV + j0 + 4 * g;
          if constexpr (sizeof(OT) == 4) {
            *reinterpret_cast<f32x4*>(dst) = acc;
          } else {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]));
          }
        }
      }
    };

    // BWD: R of block 2 cc + 1 (rows 64 + ..) for this wave's sub-block,
    // V - K S_{cc,2} with S_{cc,2} the state after the chunk's first 64 rows
    // (the snapshot of the second sub-block), in the transposed tile form of
    // the outputs: lane (i16, g) ends with row 32 a + 16 h + i16, columns
    // 4 g .. 4 g + 3.
    auto r_second = [&](int cc) {
      if (2 * cc + 1 >= bo.nb) return;
      const uint16_t* Kc = Kbuf + (cc & 1) * KELEMS;
      const uint16_t* Vc = Vbuf + (cc & 1) * C * 16;
      const float* Sn = Fsnap + (NSB / 2 - 1) * DK * 16;
      bf16x8 Sh[NKB], Sl[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(Sn + fo_f(8 * kb + 2 * g, i16));
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(Sn + fo_f(8 * kb + 2 * g + 1, i16));
        uint2 h0, l0, h1, l1;
        split4(x0, h0, l0);
        split4(x1, h1, l1);
        Sh[kb] = as_bf16x8(h0, h1);
        Sl[kb] = as_bf16x8(l0, l1);
      }
      float* rd = bblk(2 * cc + 1) + bo.r;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 32 * a + 16 * h + i16;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const bf16x8 Kh = lds16(Kc + koff<DK>(row, 4 * kb + g));
          acc = mfma16(Sh[kb], Kh, acc);
          acc = mfma16(Sl[kb], Kh, acc);
        }
        const uint2 vv = lds8(Vc + row * 16 + 4 * g);
        const f32x4 r4 = {bf16_to_f32(vv.x & 0xffffu) - acc[0], bf16_to_f32(vv.x >> 16) - acc[1],
                          bf16_to_f32(vv.y & 0xffffu) - acc[2], bf16_to_f32(vv.y >> 16) - acc[3]};
        *reinterpret_cast<f32x4*>(rd + (size_t)(row - C / 2) * DV + j0 + 4 * g) = r4;
      }
    };
    const bool bwr = BWD && a >= NSB / 2 && a < NSB;  // the waves of rows 64 ..

    // L2 prefetch: the 128-byte lines of chunk cc's k, q, v and T data are
    // split over the head's column-slice workgroups (which share an XCD and
    // its L2); output-wave thread tl touches line ct + NCT tl of the list
    // [k lines | q lines | v lines | T lines] with one dword load.  The values
    // are folded into pf_acc one chunk later, so the loads never stall
    // anything, and pf_acc is only ever stored under a condition that is
    // false.  (Whole lines rather than 64-byte sectors: the kernel runs
    // power-limited, and touching half as many lines was measured to save
    // ~3.5% of its cycles at the same clock.)  Each thread's line keeps its
    // place within the chunk, so its address is a fixed base plus the chunk
    // index times a fixed stride; on a ragged last chunk the row is clamped.
    constexpr int PFL = 128;                 // line bytes
    constexpr int LK = C * DK * 2 / PFL, LV = C * DV * 2 / PFL;
    constexpr int LT = (int)(Frag<C>::chunk_u4 * 16 / PFL);
    constexpr int NLINES = 2 * LK + LV + LT;
    static_assert(NLINES <= 256 * NCT, "one prefetch line per output-wave thread");
    const int pn = min(ct + NCT * tl, NLINES - 1);
    const char* pbase;
    size_t pstride;
    uint32_t poff, prow_bytes;
    if (pn < 2 * LK) {
      pbase = reinterpret_cast<const char*>((pn < LK ? k : q) + tokh * DK);
      pstride = (size_t)C * DK * 2;
      poff = (uint32_t)(pn % LK) * PFL;
      prow_bytes = DK * 2;
    } else if (pn < 2 * LK + LV) {
      pbase = reinterpret_cast<const char*>(v + tokh * DV);
      pstride = (size_t)C * DV * 2;
      poff = (uint32_t)(pn - 2 * LK) * PFL;
      prow_bytes = DV * 2;
    } else {
      pbase = reinterpret_cast<const char*>(Tfrag + (size_t)bh * nc * Frag<C>::chunk_u4);
      pstride = Frag<C>::chunk_u4 * 16;
      poff = (uint32_t)(pn - 2 * LK - LV) * PFL;
      prow_bytes = 0;  // T is never ragged
    }
    uint32_t pf_acc = 0, pf_val = 0;
    auto prefetch = [&](int cc) {
      uint32_t off = poff;
      if (prow_bytes && L - cc * C < C) off = min(off, (uint32_t)(L - cc * C - 1) * prow_bytes);
      pf_val = *reinterpret_cast<const uint32_t*>(pbase + (size_t)cc * pstride + off);
    };

    v_stage_load(0);
    stage_load(0);
    v_stage_store(Vbuf, 0);
    stage_store(Kbuf);
    __syncthreads();
    for (int c = 0; c < nc; ++c) {
      const int cn = min(c + 1, nc - 1);
      // ---- phase A: outputs of chunk c-1; q rows of chunk c ------------------
      stage_load(cn);
      v_stage_load(cn);
      if constexpr (BWD) {
        if (bwr && c > 0) r_second(c - 1);
      } else {
        if (outw && c > 0) outputs(c - 1);
        q_load(c);
      }
      __syncthreads();
      // ---- phase B: L2 prefetch of chunk c+2 ------------------------------------
      pf_acc ^= pf_val;
      prefetch(min(c + 2, nc - 1));
      __syncthreads();
      // ---- phase C: diagonal Q K^T block of chunk c ------------------------------
      if (!BWD && outw) diag_qk(c);
      v_stage_store(Vbuf + ((c + 1) & 1) * C * 16, (c + 1) & 1);
      stage_store(Kbuf + ((c + 1) & 1) * KELEMS);
      __syncthreads();
    }
    if constexpr (BWD) {
      if (bwr) r_second(nc - 1);
    } else {
      if (outw) outputs(nc - 1);
    }
    pf_acc ^= pf_val;
    if (nc < 0) S_final[0] = __uint_as_float(pf_acc);
  }
}

template <int C, int DK, int DV, typename OT, bool GATED, bool BWD = false>
hipError_t launch_t(const ChunkArgs& a, const uint4* Tfrag, const float* Gws) {
  using CF = Cfg<C, DK, DV>;
  const int nc = cdiv(a.L, C);
  const int BH = a.B * a.H;
  auto* kern = &scan_kernel<C, DK, DV, OT, GATED, BWD>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)CF::bytes);
  if (e != hipSuccess) return e;
  const int groups = cdiv(BH, 8) * 8 * CF::NCT;
  const BwdFwdOut bo = BWD ? *a.bwd_out : BwdFwdOut{};
  if (!BWD) prof_mark(kSlotChunkScan, false, a.stream);
  hipLaunchKernelGGL(kern, dim3(groups), dim3(CF::NTHR), CF::bytes, a.stream,
                     static_cast<const uint16_t*>(BWD ? a.k : a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), a.S0,
                     static_cast<OT*>(a.o), a.S_final, Tfrag, Gws, a.L, nc, BH, bo);
  e = hipGetLastError();
  if (!BWD) prof_mark(kSlotChunkScan, true, a.stream);
  return e;
}

template <int C, int DK, int DV>
hipError_t launch_o(const ChunkArgs& a, const uint4* Tfrag, const float* Gws) {
  if constexpr (C == 128) {
    if (a.bwd_out) return launch_t<C, DK, DV, float, false, true>(a, Tfrag, nullptr);
  }
  if (Gws)
    return a.out_dtype == 0 ? launch_t<C, DK, DV, float, true>(a, Tfrag, Gws)
                            : launch_t<C, DK, DV, bf16, true>(a, Tfrag, Gws);
  return a.out_dtype == 0 ? launch_t<C, DK, DV, float, false>(a, Tfrag, Gws)
                          : launch_t<C, DK, DV, bf16, false>(a, Tfrag, Gws);
}

template <int C>
hipError_t launch_c(const ChunkArgs& a, const uint4* Tfrag, const float* Gws) {
  if (a.d_k == 64 && a.d_v == 64) return launch_o<C, 64, 64>(a, Tfrag, Gws);
  if (a.d_k == 64 && a.d_v == 128) return launch_o<C, 64, 128>(a, Tfrag, Gws);
  if (a.d_k == 128 && a.d_v == 64) return launch_o<C, 128, 64>(a, Tfrag, Gws);
  return launch_o<C, 128, 128>(a, Tfrag, Gws);
}

}  // namespace scan

// Gws: the gated form's per-chunk log-decays, or null for the plain delta rule.
hipError_t launch_scan_mfma(const ChunkArgs& a, const uint4* Tfrag, const float* Gws) {
  return a.C == 64 ? scan::launch_c<64>(a, Tfrag, Gws) : scan::launch_c<128>(a, Tfrag, Gws);
}

}  // namespace dn
