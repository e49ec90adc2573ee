// dn_decode.hip -- single-token delta-rule decode step on gfx950.
//
// Per (b, h) the step is the layer forward at one token of the page
// "GPT-2 から Kimi K3 まで、AI モデルの進化を解説", section "DeltaNet (Fast
// weight programmers)": r = k S, u = beta (v - r), S <- S + k^T u, o = q S.
// Reading o after the write needs no second pass over S:
//     q S_new = q S + (q . k) u,
// so one streaming read of S yields both r = k S and p = q S, and S is
// written back once.  The gated step (Gated DeltaNet, article "How a Baseten
// Engineer Traced 7 Years of Attention Mechanism Evolution", Gated DeltaNet
// section: decay first, then the precise write) decays S by alpha before the
// delta reads it, which the same single read carries as scalars:
//     u = beta (v - alpha r),  o = alpha p + (q . k) u,  S <- alpha S + k^T u.  The step is bound by HBM bandwidth: per head it moves
// 2 * d_k * d_v * 4 bytes of state against 6 d_k d_v flops.
//
// Work split: persistent 512-thread workgroups, one per compute unit, each
// walking the heads bh = blockIdx.x, + gridDim.x, ...; the next head's state
// loads are issued before the current head's arithmetic, so every CU keeps one
// head's 64 KB in flight while it finishes another.  Thread (rg, cg) holds the
// float4 column group cg of rows rg, rg + ROWG, ...: a wave reads whole,
// adjacent rows, fully coalesced.  Partial r and p are reduced across row
// groups through LDS.  The updated state is written with non-temporal stores:
// it is not read again in this step, and keeping it out of the caches lets
// the write stream interleave with the read stream at a higher HBM rate
// (measured: 78% of peak for this form against 63% with one 256-thread
// workgroup per head and plain stores).
//
// Per-dimension decay (DECAY = 2; KDA as the same article describes it: the
// gate is a vector, one forgetting rate per memory dimension) decays row j of
// S by alpha[j], the key dimension a read addresses.  The single read then
// carries k o alpha and q o alpha:
//     u = beta (v - (k o alpha) S),  o = (q o alpha) S + (q . k) u,
//     S <- diag(alpha) S + k^T u.
//
// With FEAT the step also applies the layer's feature maps to its inputs
// (same page and section: q, k = normalise(silu(.)), beta = sigmoid(logit);
// dn_features.h): waves 0 and 1 map k and q while waves 2 and 3 stage v, and
// the mapped q, k are held in the input dtype, as the streaming feature
// kernel stores them for the chunked path.  It adds no memory traffic.

#include "dn_common.h"
#include "dn_features.h"
#include "dn_launch.h"

namespace dn {

typedef float vf4 __attribute__((ext_vector_type(4)));

// One head's q or k row through the feature maps by one wave: silu, the
// row's norm by a wave reduction, the scaled values rounded to the input
// dtype, into LDS.
template <int DK, typename IT>
__device__ __forceinline__ void map_row_to_lds(const IT* __restrict__ x, float* dst, int lane) {
  constexpr int E = DK / 64;
  float f[E];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    f[e] = fast_silu(to_f32(x[lane + 64 * e]));
    ss += f[e] * f[e];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float r = inv_row_norm(ss);
#pragma unroll
  for (int e = 0; e < E; ++e) dst[lane + 64 * e] = to_f32(from_f32<IT>(f[e] * r));
}

// DECAY: 0 none, 1 one alpha per (b, h), 2 one alpha per key dimension.
template <int DK, int DV, typename IT, typename OT, int DECAY, bool FEAT>
__global__ __launch_bounds__(512) void decode_step_kernel(
    const IT* __restrict__ q, const IT* __restrict__ k, const IT* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, float* __restrict__ S,
    OT* __restrict__ o, int BH) {
  constexpr int NT = 512;
  constexpr int COLG = DV / 4;          // float4 column groups per row
  constexpr int ROWG = NT / COLG;       // row groups
  constexpr int RPT = DK / ROWG;        // rows per thread
  static_assert(RPT * ROWG == DK && COLG * ROWG == NT, "tile shape");
  constexpr bool GATED = DECAY == 1, PERDIM = DECAY == 2;

  __shared__ float ks[DK], qs[DK], vs[DV], us[DV];
  __shared__ float ad[PERDIM ? DK : 1];  // per-dimension decays
  __shared__ vf4 red_r[ROWG][COLG], red_p[ROWG][COLG];
  __shared__ float qk_s;

  const int tid = threadIdx.x;
  const int cg = tid % COLG, rg = tid / COLG;
  auto load_state = [&](int bh, vf4 (&dst)[RPT]) {
    const float* Sh = S + (size_t)bh * (DK * DV);
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      dst[i] = *reinterpret_cast<const vf4*>(Sh + (size_t)(rg + i * ROWG) * DV + cg * 4);
  };

  int bh = blockIdx.x;
  if (bh >= BH) return;
  // The states of this head and of the next two, in flight meanwhile.
  auto next_of = [&](int h) {  // no int overflow near BH = 2^31
    const long long nl = (long long)h + gridDim.x;
    return nl < BH ? (int)nl : h;
  };
  vf4 s[RPT], sn[RPT], snn[RPT];
  load_state(bh, s);
  int nb = next_of(bh);
  load_state(nb, sn);
  for (;;) {
    const bool more = nb != bh;
    const int nnb = next_of(nb);
    load_state(nnb, snn);
    if (FEAT) {
      static_assert(DK % 64 == 0, "one wave per feature row");
      static_assert(128 + DV <= NT, "v staged by the waves that do not map");
      if (tid < 64)
        map_row_to_lds<DK>(k + (size_t)bh * DK, ks, tid);
      else if (tid < 128)
        map_row_to_lds<DK>(q + (size_t)bh * DK, qs, tid - 64);
      else if (tid < 128 + DV)  // waves 2.. stage v, so its load overlaps the maps
        vs[tid - 128] = to_f32(v[(size_t)bh * DV + tid - 128]);
    } else {
      for (int i = tid; i < DK; i += NT) {
        ks[i] = to_f32(k[(size_t)bh * DK + i]);
        qs[i] = to_f32(q[(size_t)bh * DK + i]);
      }
      for (int i = tid; i < DV; i += NT) vs[i] = to_f32(v[(size_t)bh * DV + i]);
    }
    if (PERDIM)
      for (int i = tid; i < DK; i += NT) ad[i] = alpha[(size_t)bh * DK + i];
    __syncthreads();

    if (tid < 64) {  // q . k by one wave
      float acc = 0.f;
      for (int i = tid; i < DK; i += 64) acc += qs[i] * ks[i];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
      if (tid == 0) qk_s = acc;
    }

    vf4 r = 0.f, p = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg + i * ROWG;
      const float dr = PERDIM ? ad[row] : 1.f;
      r += (ks[row] * dr) * s[i];
      p += (qs[row] * dr) * s[i];
    }
    red_r[rg][cg] = r;
    red_p[rg][cg] = p;
    __syncthreads();

    const float b = FEAT ? fast_sigmoid(beta[bh]) : beta[bh];
    const float al = GATED ? alpha[bh] : 1.f;
    for (int c = tid; c < DV; c += NT) {
      const int g = c / 4, e = c % 4;
      float rr = 0.f, pp = 0.f;
#pragma unroll
      for (int j = 0; j < ROWG; ++j) {
        rr += red_r[j][g][e];
        pp += red_p[j][g][e];
      }
      const float u = GATED ? b * (vs[c] - al * rr) : b * (vs[c] - rr);
      us[c] = u;
      o[(size_t)bh * DV + c] = from_f32<OT>(GATED ? al * pp + qk_s * u : pp + qk_s * u);
    }
    __syncthreads();

    const vf4 u4 = *reinterpret_cast<const vf4*>(&us[cg * 4]);
    float* Sh = S + (size_t)bh * (DK * DV);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg + i * ROWG;
      const vf4 snew = GATED    ? al * s[i] + ks[row] * u4
                       : PERDIM ? ad[row] * s[i] + ks[row] * u4
                                : s[i] + ks[row] * u4;
      __builtin_nontemporal_store(snew, reinterpret_cast<vf4*>(Sh + (size_t)row * DV + cg * 4));
    }
    __syncthreads();  // the LDS vectors are rewritten for the next head
    if (!more) break;
    bh = nb;
    nb = nnb;
    for (int i = 0; i < RPT; ++i) s[i] = sn[i], sn[i] = snn[i];
  }
}

// Compute units of the current device (the persistent grid size), cached per
// device.
static int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

template <int DK, int DV, typename IT, typename OT>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  const int BH = a.B * a.H;
  const int grid = BH < cu_count() ? BH : cu_count();
  prof_mark(kSlotDecode, false, a.stream);
  const IT *q = static_cast<const IT*>(a.q), *k = static_cast<const IT*>(a.k);
  const IT* v = static_cast<const IT*>(a.v);
  OT* o = static_cast<OT*>(a.o);
  const dim3 g(grid), blk(512);
  const int decay = a.alpha ? (a.per_dim_alpha ? 2 : 1) : 0;
#define DN_DECODE_LAUNCH(D, F)                                                                \
  hipLaunchKernelGGL((decode_step_kernel<DK, DV, IT, OT, D, F>), g, blk, 0, a.stream, q, k, v, \
                     a.alpha, a.beta, a.S, o, BH)
  if (a.features) {
    if (decay == 2) DN_DECODE_LAUNCH(2, true);
    else if (decay == 1) DN_DECODE_LAUNCH(1, true);
    else DN_DECODE_LAUNCH(0, true);
  } else {
    if (decay == 2) DN_DECODE_LAUNCH(2, false);
    else if (decay == 1) DN_DECODE_LAUNCH(1, false);
    else DN_DECODE_LAUNCH(0, false);
  }
#undef DN_DECODE_LAUNCH
  hipError_t e = hipGetLastError();
  prof_mark(kSlotDecode, true, a.stream);
  return e;
}

template <int DK, int DV>
static hipError_t launch_decode_d(const DecodeArgs& a) {
  if (a.in_dtype == 0 && a.out_dtype == 0) return launch_decode_t<DK, DV, float, float>(a);
  if (a.in_dtype == 0 && a.out_dtype == 1) return launch_decode_t<DK, DV, float, bf16>(a);
  if (a.in_dtype == 1 && a.out_dtype == 0) return launch_decode_t<DK, DV, bf16, float>(a);
  return launch_decode_t<DK, DV, bf16, bf16>(a);
}

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.d_k == 64 && a.d_v == 64) return launch_decode_d<64, 64>(a);
  if (a.d_k == 64 && a.d_v == 128) return launch_decode_d<64, 128>(a);
  if (a.d_k == 128 && a.d_v == 64) return launch_decode_d<128, 64>(a);
  return launch_decode_d<128, 128>(a);
}

}  // namespace dn
