// Codebook update of one Lloyd iteration of plain (unweighted) k-means on the
// coupled vectors of a layer.
//
// What it computes [LoopVQ paper, hub.valency.io/works/W_7srt5hed_v1,
// section "Redundancy along the loop axis", Fig. 2c: plain k-means with the
// loop-axis grouping of eq. (4) against a grouping of G channels of one
// step]: the assignment half of an iteration is the encoder's nearest-entry
// rule (loopvq_encode writes the codes); this half moves every entry to the
// mean of the coupled vectors coded with it (an entry with no vectors keeps
// its value), rounded to fp16, and sums the reconstruction error
// ||z - e_code||^2 and ||z||^2 of every (block, head, K|V) stream.
//
// MI355X mapping: a workgroup takes a range of tokens of one stream; each
// thread takes one coupled vector at a time (its code from the index row, its
// G values as Tc runs of c channels), adds it into per-entry fp64 sums in LDS
// (ds_add_f64) and counts the entry, and the workgroup then adds its LDS sums
// into the stream's fp64 sums in global memory.  fp64 sums of bf16 or fp16
// values are exact, so the result does not depend on the order of the adds.
// A second kernel divides and rounds.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace loopvq {

__global__ void kmeans_zero_kernel(double* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0.0;
}

template <int G, bool XF32>
__global__ __launch_bounds__(256) void kmeans_accum_kernel(KmeansParams p) {
  // per-entry sums with rows of G + 1 doubles (the odd stride spreads the random
  // entries of a wave over the LDS banks), then [K] counts and [2] error sums
  constexpr int GS = G + 1;
  __shared__ double kms[256 * GS + 256 + 2];
  const int K = p.K, H = p.H_kv, C = p.c, Tc = p.Tc, D = p.D;
  double* s_sum = kms;
  double* s_cnt = kms + (size_t)K * GS;
  double* s_err = s_cnt + K;
  for (int i = threadIdx.x; i < K * GS + K + 2; i += blockDim.x) kms[i] = 0.0;
  __syncthreads();

  const int y = blockIdx.y;                  // stream (beta*2 + kv)*H + h of this call
  const int h = y % H, kv = (y / H) & 1, beta = y / (2 * H);
  const int n = D / C;
  const int P = 1 << p.log2P;
  const int R = n * p.bits / 8;
  const void* x = kv ? p.xv : p.xk;
  const uint16_t* cb = p.cb + ((size_t)(beta * H + h) * 2 + kv) * K * G;
  const uint8_t* cache = p.cache + (int64_t)beta * p.block_stride;
  const int t0 = blockIdx.x * p.tok_per_wg, t1 = min(t0 + p.tok_per_wg, p.n_tok);
  double err = 0.0, nrm = 0.0;
  for (int v = t0 * n + threadIdx.x; v < t1 * n; v += blockDim.x) {
    const int tok = v / n, g = v - tok * n;
    const int slot = p.slot_mapping[tok];
    const uint8_t* row = cache + ((((size_t)(slot >> p.log2P) * H + h) * 2 + kv) * P + (slot & (P - 1))) * R;
    const int sl = row_slot_of_group(g, n);
    int code;
    if (p.bits == 8) code = row[sl];
    else code = (row[sl >> 1] >> ((sl & 1) * 4)) & 15;
    const uint16_t* e = cb + (size_t)code * G;
    double* acc = s_sum + (size_t)code * GS;
    for (int m = 0; m < Tc; ++m) {
      const size_t off = (((size_t)(beta * Tc + m) * p.n_tok + tok) * H + h) * D + (size_t)g * C;
      for (int i = 0; i < C; ++i) {
        double z;
        if constexpr (XF32) z = (double)((const float*)x)[off + i];
        else z = (double)u2f((uint32_t)((const uint16_t*)x)[off + i] << 16);
        const double d = z - (double)__builtin_bit_cast(_Float16, e[i * Tc + m]);
        err = fma(d, d, err);
        nrm = fma(z, z, nrm);
        atomicAdd(acc + i * Tc + m, z);
      }
    }
    atomicAdd(s_cnt + code, 1.0);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    err += __shfl_xor(err, o);
    nrm += __shfl_xor(nrm, o);
  }
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(s_err, err);
    atomicAdd(s_err + 1, nrm);
  }
  __syncthreads();
  double* gsum = p.gsum + (size_t)y * (K * G + K + 2);
  for (int i = threadIdx.x; i < K * G + K + 2; i += blockDim.x) {
    const double v = i < K * G ? kms[(i / G) * GS + i % G] : kms[K * GS + (i - K * G)];
    if (v != 0.0) atomicAdd(gsum + i, v);
  }
}

// entry e of stream y: mean of its vectors rounded to fp16, or unchanged
__global__ void kmeans_finalize_kernel(KmeansParams p, int G, int n_streams) {
  const int K = p.K, H = p.H_kv;
  const size_t total = (size_t)n_streams * K * G;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int y = (int)(i / ((size_t)K * G));
    const int r = (int)(i - (size_t)y * K * G);
    const int e = r / G;
    const int h = y % H, kv = (y / H) & 1, beta = y / (2 * H);
    const size_t ci = (((size_t)(beta * H + h) * 2 + kv) * K) * G + r;
    const double* gs = p.gsum + (size_t)y * (K * G + K + 2);
    const double cnt = gs[(size_t)K * G + e];
    p.cb_out[ci] = cnt > 0.0 ? __builtin_bit_cast(uint16_t, (_Float16)(gs[r] / cnt)) : p.cb[ci];
    if (r == 0 && p.err != nullptr) {
      const size_t eo = (((size_t)(beta * H + h) * 2 + kv)) * 2;
      p.err[eo] = gs[(size_t)K * G + K];
      p.err[eo + 1] = gs[(size_t)K * G + K + 1];
    }
  }
}

hipError_t launch_kmeans_update(bool xf32, const KmeansParams& p, int n_blocks, hipStream_t s) {
  const int G = p.c * p.Tc;
  const int n_streams = n_blocks * 2 * p.H_kv;
  const size_t per = (size_t)p.K * G + p.K + 2;
  const size_t nz = per * n_streams;
  hipLaunchKernelGGL(kmeans_zero_kernel, dim3((unsigned)std::min<size_t>((nz + 255) / 256, 4096)), dim3(256), 0, s,
                     p.gsum, nz);
  if (p.n_tok > 0) {
    const dim3 grid((p.n_tok + p.tok_per_wg - 1) / p.tok_per_wg, n_streams);
#define LVQ_KM(g)                                                                                  \
    if (G == g) {                                                                                  \
      if (xf32) hipLaunchKernelGGL((kmeans_accum_kernel<g, true>), grid, dim3(256), 0, s, p);     \
      else hipLaunchKernelGGL((kmeans_accum_kernel<g, false>), grid, dim3(256), 0, s, p);         \
    }
    LVQ_KM(8) LVQ_KM(16) LVQ_KM(32)
#undef LVQ_KM
  }
  const size_t tot = (size_t)n_streams * p.K * G;
  hipLaunchKernelGGL(kmeans_finalize_kernel, dim3((unsigned)std::min<size_t>((tot + 255) / 256, 4096)), dim3(256), 0,
                     s, p, G, n_streams);
  return hipGetLastError();
}

}  // namespace loopvq
