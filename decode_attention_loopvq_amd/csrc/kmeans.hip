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
// G values as Tc runs of c channels, one vector load per run), adds it into
// per-entry fp64 sums in LDS (ds_add_f64), counts the entry and sums ||z||^2,
// and the workgroup then adds its LDS sums into the stream's fp64 sums in
// global memory.  fp64 sums of bf16 or fp16 values are exact, so the result
// does not depend on the order of the adds.  A second kernel, one workgroup
// per stream, divides and rounds, and forms the error from the same sums:
// sum_v ||z_v - e_code(v)||^2 = sum_v ||z_v||^2 - 2 sum_r e_r . S_r
// + sum_r n_r ||e_r||^2 with S_r and n_r the sum and count of entry r, so the
// first kernel never reads the codebook.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace loopvq {

__global__ void kmeans_zero_kernel(double* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0.0;
}

// the C channels of one loop step of a coupled vector, as floats
template <int C, bool XF32>
__device__ __forceinline__ void load_channels(const void* x, size_t off, float* z) {
  if constexpr (XF32) {
    const float* s = (const float*)x + off;
    if constexpr (C == 2) {
      const float2v a = *(const float2v*)s;
      z[0] = a.x; z[1] = a.y;
    } else {
#pragma unroll
      for (int j = 0; j < C / 4; ++j) {
        const float4v a = *(const float4v*)(s + 4 * j);
        z[4 * j] = a.x; z[4 * j + 1] = a.y; z[4 * j + 2] = a.z; z[4 * j + 3] = a.w;
      }
    }
  } else {
    const uint16_t* s = (const uint16_t*)x + off;
    uint32_t w[C / 2];
    if constexpr (C == 2) {
      w[0] = *(const uint32_t*)s;
    } else if constexpr (C == 4) {
      const uint2v a = *(const uint2v*)s;
      w[0] = a.x; w[1] = a.y;
    } else {
#pragma unroll
      for (int j = 0; j < C / 8; ++j) {
        const uint4v a = *(const uint4v*)(s + 8 * j);
        w[4 * j] = a.x; w[4 * j + 1] = a.y; w[4 * j + 2] = a.z; w[4 * j + 3] = a.w;
      }
    }
#pragma unroll
    for (int i = 0; i < C; ++i) z[i] = (i & 1) ? bf16hi(w[i >> 1]) : bf16lo(w[i >> 1]);
  }
}

template <int G, int C, bool XF32>
__global__ __launch_bounds__(256) void kmeans_accum_kernel(KmeansParams p) {
  // per-entry sums with rows of G + 1 doubles (the odd stride spreads the random
  // entries of a wave over the LDS banks), then [K] counts and [2] (unused, ||z||^2)
  constexpr int GS = G + 1;
  constexpr int TC = G / C;
  __shared__ double kms[256 * GS + 256 + 2];
  const int K = p.K, H = p.H_kv, D = p.D;
  double* s_sum = kms;
  double* s_cnt = kms + (size_t)K * GS;
  double* s_nrm = s_cnt + K + 1;
  for (int i = threadIdx.x; i < K * GS + K + 2; i += blockDim.x) kms[i] = 0.0;
  __syncthreads();

  const int y = blockIdx.y;                  // stream (beta*2 + kv)*H + h of this call
  const int h = y % H, kv = (y / H) & 1, beta = y / (2 * H);
  const int n = D / C;
  const int P = 1 << p.log2P;
  const int R = n * p.bits / 8;
  const void* x = kv ? p.xv : p.xk;
  const uint8_t* cache = p.cache + (int64_t)beta * p.block_stride;
  const int t0 = blockIdx.x * p.tok_per_wg, t1 = min(t0 + p.tok_per_wg, p.n_tok);
  double nrm = 0.0;
  for (int v = t0 * n + threadIdx.x; v < t1 * n; v += blockDim.x) {
    const int tok = v / n, g = v - tok * n;
    const int slot = p.slot_mapping[tok];
    const uint8_t* row = cache + ((((size_t)(slot >> p.log2P) * H + h) * 2 + kv) * P + (slot & (P - 1))) * R;
    const int sl = row_slot_of_group(g, n);
    int code;
    if (p.bits == 8) code = row[sl];
    else code = (row[sl >> 1] >> ((sl & 1) * 4)) & 15;
    double* acc = s_sum + (size_t)code * GS;
#pragma unroll
    for (int m = 0; m < TC; ++m) {
      float z[C];
      load_channels<C, XF32>(x, (((size_t)(beta * TC + m) * p.n_tok + tok) * H + h) * D + (size_t)g * C, z);
#pragma unroll
      for (int i = 0; i < C; ++i) {
        const double zd = (double)z[i];
        nrm = fma(zd, zd, nrm);
        atomicAdd(acc + i * TC + m, zd);
      }
    }
    atomicAdd(s_cnt + code, 1.0);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nrm += __shfl_xor(nrm, o);
  if ((threadIdx.x & 63) == 0) atomicAdd(s_nrm, nrm);
  __syncthreads();
  double* gsum = p.gsum + (size_t)y * (K * G + K + 2);
  for (int i = threadIdx.x; i < K * G + K + 2; i += blockDim.x) {
    const double v = i < K * G ? kms[(i / G) * GS + i % G] : kms[K * GS + (i - K * G)];
    if (v != 0.0) atomicAdd(gsum + i, v);
  }
}

// one workgroup per stream y: entry e becomes the mean of its vectors rounded to
// fp16, or stays unchanged; the stream's error and ||z||^2 sums are written
__global__ __launch_bounds__(1024) void kmeans_finalize_kernel(KmeansParams p, int G) {
  __shared__ double red[16];
  const int K = p.K, H = p.H_kv;
  const int y = blockIdx.x;
  const int h = y % H, kv = (y / H) & 1, beta = y / (2 * H);
  const size_t c0 = (((size_t)(beta * H + h) * 2 + kv) * K) * G;
  const double* gs = p.gsum + (size_t)y * (K * G + K + 2);
  double part = 0.0;                        // sum_r n_r ||e_r||^2 - 2 e_r . S_r
  for (int r = threadIdx.x; r < K * G; r += blockDim.x) {
    const double cnt = gs[(size_t)K * G + r / G];
    const uint16_t old = p.cb[c0 + r];
    const double e = (double)__builtin_bit_cast(_Float16, old);
    part = fma(e, fma(cnt, e, -2.0 * gs[r]), part);
    p.cb_out[c0 + r] = cnt > 0.0 ? __builtin_bit_cast(uint16_t, (_Float16)(gs[r] / cnt)) : old;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
  __syncthreads();
  if (threadIdx.x == 0 && p.err != nullptr) {
    double tot = 0.0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += red[w];
    const double nrm = gs[(size_t)K * G + K + 1];
    const size_t eo = (((size_t)(beta * H + h) * 2 + kv)) * 2;
    p.err[eo] = nrm + tot;
    p.err[eo + 1] = nrm;
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
#define LVQ_KM(GG, CC)                                                                                  \
    if (G == GG && p.c == CC) {                                                                         \
      if (xf32) hipLaunchKernelGGL((kmeans_accum_kernel<GG, CC, true>), grid, dim3(256), 0, s, p);     \
      else hipLaunchKernelGGL((kmeans_accum_kernel<GG, CC, false>), grid, dim3(256), 0, s, p);         \
    }
    LVQ_KM(8, 2) LVQ_KM(8, 4) LVQ_KM(8, 8)
    LVQ_KM(16, 2) LVQ_KM(16, 4) LVQ_KM(16, 8) LVQ_KM(16, 16)
    LVQ_KM(32, 2) LVQ_KM(32, 4) LVQ_KM(32, 8)
#undef LVQ_KM
  }
  hipLaunchKernelGGL(kmeans_finalize_kernel, dim3(n_streams), dim3(1024), 0, s, p, G);
  return hipGetLastError();
}

}  // namespace loopvq
