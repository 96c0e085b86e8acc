// TaSQ key transform ahead of LoopVQ coding (TaSQ+LoopVQ).
//
// What it computes [LoopVQ paper, hub.valency.io/works/W_7srt5hed_v1,
// appendix "Orthogonal application with TaSQ", "Formulation" and "Grouping
// under loop coupling"; "Calibration and bitwidth" for the fp16 scale]: for
// loop step t, token j and KV head h, u = P(w (.) k / sigma_j), where w are the
// channel weights of (t, h), sigma_j the root mean square of w (.) k over all
// heads and channels of token j at step t, kept in fp16, and P the pair
// permutation of the step's block: u channel 2p holds key channel perm[p] and
// u channel 2p+1 holds perm[p] + D/2, so a code of c consecutive u channels
// covers c/2 whole RoPE pairs.  The coupled vectors of the keys are then built
// from u as they would be from k.  A token whose fp16 sigma is 0 gets u = 0.
//
// MI355X mapping: one wave per (token, loop step), four per workgroup.  The
// wave reads the token's H*D inputs in 16-byte runs, sums the weighted squares
// in fp64 (the sum then matches an exact evaluation except within fp64
// rounding of an fp16 rounding midpoint) and reduces across lanes with
// shuffles; every lane then holds sigma.  u is formed in fp64 as w k * (1 /
// sigma) and rounded to fp32; each lane writes 8 consecutive u channels (4
// RoPE pairs of one head) as two 16-byte stores, reading their inputs at the
// permuted positions (cached: the wave has just read the token's row).  The
// pass is bound by HBM bandwidth (6 bytes per bf16 element).
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace loopvq {

template <bool XF32>
__device__ __forceinline__ double load_x(const void* x, size_t i) {
  if constexpr (XF32) return (double)((const float*)x)[i];
  else return (double)u2f((uint32_t)((const uint16_t*)x)[i] << 16);
}

template <bool XF32>
__global__ __launch_bounds__(256) void tasq_transform_kernel(TasqParams p) {
  const int lane = threadIdx.x & 63;
  const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);   // token-major within a step
  if (item >= (long long)p.n_tok * p.n_steps) return;                      // whole waves exit together
  const int s = (int)(item / p.n_tok), j = (int)(item - (long long)s * p.n_tok);
  const int step = p.first_step + s;
  const int D = p.D, D2 = p.D / 2, HD = p.H * p.D;
  const float* w = p.w + (size_t)step * HD;
  const int32_t* perm = p.perm + (size_t)(step / p.Tc) * p.H * D2;
  const size_t xoff = ((size_t)s * p.n_tok + j) * HD;

  // sum of (w k)^2 over the token's H*D values, 8 consecutive values per lane and pass
  double acc = 0.0;
  for (int e0 = lane * 8; e0 < HD; e0 += 512) {
    float x[8];
    if constexpr (XF32) {
      const float4v a = *(const float4v*)((const float*)p.xk + xoff + e0);
      const float4v b = *(const float4v*)((const float*)p.xk + xoff + e0 + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
      const uint4v a = *(const uint4v*)((const uint16_t*)p.xk + xoff + e0);
      const uint32_t wd[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) { x[2 * i] = bf16lo(wd[i]); x[2 * i + 1] = bf16hi(wd[i]); }
    }
    const float4v wa = *(const float4v*)(w + e0), wb = *(const float4v*)(w + e0 + 4);
    const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double y = (double)x[i] * (double)wv[i];
      acc = fma(y, y, acc);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  const _Float16 s16 = (_Float16)(float)sqrt(acc / (double)HD);
  if (lane == 0) p.sigma[(size_t)step * p.sigma_stride + p.slot_mapping[j]] = __builtin_bit_cast(uint16_t, s16);
  const double inv = (float)s16 > 0.f ? 1.0 / (double)(float)s16 : 0.0;

  // u channels e0 .. e0+7 (pairs (e0 % D)/2 .. +3 of head e0 / D)
  for (int e0 = lane * 8; e0 < HD; e0 += 512) {
    const int h = e0 / D, p0 = (e0 - h * D) >> 1;
    float u[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int f = min(max(perm[h * D2 + p0 + r], 0), D2 - 1);
      const int cf = h * D + f, ch = cf + D2;
      u[2 * r] = (float)(load_x<XF32>(p.xk, xoff + cf) * (double)w[cf] * inv);
      u[2 * r + 1] = (float)(load_x<XF32>(p.xk, xoff + ch) * (double)w[ch] * inv);
    }
    float* dst = p.u + xoff + e0;
    *(float4v*)dst = (float4v){u[0], u[1], u[2], u[3]};
    *(float4v*)(dst + 4) = (float4v){u[4], u[5], u[6], u[7]};
  }
}

hipError_t launch_tasq_transform(bool xf32, const TasqParams& p, int n_steps, hipStream_t s) {
  const long long items = (long long)p.n_tok * n_steps;
  if (items == 0) return hipSuccess;
  TasqParams q = p;
  q.n_steps = n_steps;
  const dim3 grid((unsigned)((items + 3) / 4));
  if (xf32) hipLaunchKernelGGL(tasq_transform_kernel<true>, grid, dim3(256), 0, s, q);
  else hipLaunchKernelGGL(tasq_transform_kernel<false>, grid, dim3(256), 0, s, q);
  return hipGetLastError();
}

}  // namespace loopvq
