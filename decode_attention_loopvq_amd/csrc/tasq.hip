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
// MI355X mapping: one workgroup of 256 threads per (token, loop step).  The
// weighted squares are summed in fp64 (the sum then matches an exact
// evaluation except within fp64 rounding of an fp16 rounding midpoint), the
// block reduction goes through DPP-free shuffles and LDS, and u is formed in
// fp64 from the fp16 sigma and rounded once to fp32.  The pass reads the
// token's H*D inputs twice (the second time from cache) and writes u in u
// order (coalesced); it is bound by HBM bandwidth.
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
  __shared__ double red[4];
  __shared__ float sig;
  const int j = blockIdx.x, s = blockIdx.y;
  const int step = p.first_step + s;
  const int D = p.D, D2 = p.D / 2, HD = p.H * p.D;
  const float* w = p.w + (size_t)step * HD;
  const int32_t* perm = p.perm + (size_t)(step / p.Tc) * p.H * D2;
  const size_t xoff = ((size_t)s * p.n_tok + j) * HD;

  double acc = 0.0;
  for (int e = threadIdx.x; e < HD; e += 256) {
    const double y = load_x<XF32>(p.xk, xoff + e) * (double)w[e];
    acc = fma(y, y, acc);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double ms = (red[0] + red[1] + red[2] + red[3]) / (double)HD;
    const _Float16 s16 = (_Float16)(float)sqrt(ms);
    sig = (float)s16;
    p.sigma[(size_t)step * p.sigma_stride + p.slot_mapping[j]] = __builtin_bit_cast(uint16_t, s16);
  }
  __syncthreads();
  const double sd = (double)sig;
  for (int e = threadIdx.x; e < HD; e += 256) {
    const int h = e / D, cc = e - h * D;
    const int f = min(max(perm[h * D2 + (cc >> 1)], 0), D2 - 1) + (cc & 1) * D2;
    const double y = load_x<XF32>(p.xk, xoff + (size_t)h * D + f) * (double)w[h * D + f];
    p.u[xoff + e] = sd > 0.0 ? (float)(y / sd) : 0.f;
  }
}

hipError_t launch_tasq_transform(bool xf32, const TasqParams& p, int n_steps, hipStream_t s) {
  if (p.n_tok == 0 || n_steps == 0) return hipSuccess;
  const dim3 grid(p.n_tok, n_steps);
  if (xf32) hipLaunchKernelGGL(tasq_transform_kernel<true>, grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL(tasq_transform_kernel<false>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace loopvq
