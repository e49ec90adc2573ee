// dn_decode.hip -- single-token delta-rule decode step on gfx950.
//
// Per (b, h) the step is the layer forward at one token of the page
// "GPT-2 から Kimi K3 まで、AI モデルの進化を解説", section "DeltaNet (Fast
// weight programmers)": r = k S, u = beta (v - r), S <- S + k^T u, o = q S.
// Reading o after the write needs no second pass over S:
//     q S_new = q S + (q . k) u,
// so one streaming read of S yields both r = k S and p = q S, and S is
// written back once.  The step is bound by HBM bandwidth: per head it moves
// 2 * d_k * d_v * 4 bytes of state against 6 d_k d_v flops.
//
// Work split: one 256-thread workgroup per (b, h).  Thread (rg, cg) holds a
// float4 column group cg of the rows rg, rg + ROWG, rg + 2 ROWG, ...; a wave
// therefore reads whole, adjacent 512-byte rows (d_v = 128), fully
// coalesced.  Partial r and p are reduced across row groups through LDS.

#include "dn_common.h"
#include "dn_launch.h"

namespace dn {

template <int DK, int DV, typename IT, typename OT>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const IT* __restrict__ q, const IT* __restrict__ k, const IT* __restrict__ v,
    const float* __restrict__ beta, float* __restrict__ S, OT* __restrict__ o) {
  constexpr int COLG = DV / 4;          // float4 column groups per row
  constexpr int ROWG = 256 / COLG;      // row groups
  constexpr int RPT = DK / ROWG;        // rows per thread
  static_assert(RPT * ROWG == DK && COLG * ROWG == 256, "tile shape");

  __shared__ float ks[DK], qs[DK], vs[DV], us[DV];
  __shared__ float4 red_r[ROWG][COLG], red_p[ROWG][COLG];
  __shared__ float qk_s;

  const int tid = threadIdx.x;
  const size_t bh = blockIdx.x;
  const int cg = tid % COLG, rg = tid / COLG;
  float* Sh = S + bh * (size_t)(DK * DV);

  // Issue the state loads first; they dominate the step's latency.
  float4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + i * ROWG;
    s[i] = *reinterpret_cast<const float4*>(Sh + (size_t)row * DV + cg * 4);
  }
  for (int i = tid; i < DK; i += 256) {
    ks[i] = to_f32(k[bh * DK + i]);
    qs[i] = to_f32(q[bh * DK + i]);
  }
  for (int i = tid; i < DV; i += 256) vs[i] = to_f32(v[bh * DV + i]);
  __syncthreads();

  if (tid < 64) {  // q . k by one wave
    float acc = 0.f;
    for (int i = tid; i < DK; i += 64) acc += qs[i] * ks[i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (tid == 0) qk_s = acc;
  }

  float4 r = make_float4(0.f, 0.f, 0.f, 0.f), p = r;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + i * ROWG;
    const float kr = ks[row], qr = qs[row];
    r.x += kr * s[i].x; r.y += kr * s[i].y; r.z += kr * s[i].z; r.w += kr * s[i].w;
    p.x += qr * s[i].x; p.y += qr * s[i].y; p.z += qr * s[i].z; p.w += qr * s[i].w;
  }
  red_r[rg][cg] = r;
  red_p[rg][cg] = p;
  __syncthreads();

  const float b = beta[bh];
  for (int c = tid; c < DV; c += 256) {
    const int g = c / 4, e = c % 4;
    float rr = 0.f, pp = 0.f;
#pragma unroll
    for (int j = 0; j < ROWG; ++j) {
      const float* pr = reinterpret_cast<const float*>(&red_r[j][g]);
      const float* pq = reinterpret_cast<const float*>(&red_p[j][g]);
      rr += pr[e];
      pp += pq[e];
    }
    const float u = b * (vs[c] - rr);
    us[c] = u;
    o[bh * DV + c] = from_f32<OT>(pp + qk_s * u);
  }
  __syncthreads();

  const float4 u4 = *reinterpret_cast<const float4*>(&us[cg * 4]);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + i * ROWG;
    const float kr = ks[row];
    float4 t = s[i];
    t.x += kr * u4.x; t.y += kr * u4.y; t.z += kr * u4.z; t.w += kr * u4.w;
    *reinterpret_cast<float4*>(Sh + (size_t)row * DV + cg * 4) = t;
  }
}

template <int DK, int DV, typename IT, typename OT>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  prof_mark(kSlotDecode, false, a.stream);
  hipLaunchKernelGGL((decode_step_kernel<DK, DV, IT, OT>), dim3(a.B * a.H), dim3(256), 0,
                     a.stream, static_cast<const IT*>(a.q), static_cast<const IT*>(a.k),
                     static_cast<const IT*>(a.v), a.beta, a.S, static_cast<OT*>(a.o));
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
