// Combine kernel and the split-kernel launchers (shared codebooks).  The
// split kernel itself is in decode_split.h.
#include "decode_split.h"

namespace loopvq {

// ---- combine: one workgroup per (request, query head).  The partials are
//      the chunks of the coded positions and, when given, one partial over
//      the request's bf16 tokens (sink and recent window); all are merged by
//      their log-sum-exp.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void decode_combine_kernel(CombineParams p) {
  constexpr int SETS = 256 / D;          // partial subsets processed side by side
  __shared__ float red_m[256];
  __shared__ float red_o[256];
  __shared__ float red_w[SETS];
  const int pq = blockIdx.x;
  const int b = pq / p.H_q, jq = pq - b * p.H_q;
  const int h = jq / p.grp, k = b * p.grp + (jq - h * p.grp);
  const int len = min(max(p.seq_lens[b], 0), p.max_seq_len);
  const int npart = len > 0 ? (len + p.Lc - 1) / p.Lc : 0;
  const size_t base = (size_t)(h * p.n_pairs + k) * p.n_chunks;
  const int tid = threadIdx.x;
  const size_t wpart = (size_t)h * p.n_pairs + k;
  const float wle = p.win_lse != nullptr ? p.win_lse[wpart] : -INFINITY;
  float M = tid == 0 ? wle : -INFINITY;
  for (int i = tid; i < npart; i += 256) M = fmaxf(M, p.part_lse[base + i]);
  red_m[tid] = M;
  __syncthreads();
  for (int sft = 128; sft > 0; sft >>= 1) {
    if (tid < sft) red_m[tid] = fmaxf(red_m[tid], red_m[tid + sft]);
    __syncthreads();
  }
  M = red_m[0];
  const int set = tid / D, d = tid - set * D;
  float o = 0.f, W = 0.f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int i = set; i < npart; i += SETS) {
      const float le = p.part_lse[base + i];
      const float w = le == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(le - M);
      W += w;
      o = fmaf(w, p.part_o[(base + i) * D + d], o);
    }
    if (set == 0 && wle != -INFINITY) {
      const float w = __builtin_amdgcn_exp2f(wle - M);
      W += w;
      o = fmaf(w, p.win_o[wpart * D + d], o);
    }
  }
  red_o[tid] = o;
  if (d == 0) red_w[set] = W;
  __syncthreads();
  if (set == 0) {
    float Wt = 0.f, ot = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < SETS; ++s2) { Wt += red_w[s2]; ot += red_o[s2 * D + d]; }
    const float v = Wt > 0.f ? ot / Wt : 0.f;
    const size_t oo = (size_t)pq * D + d;
    if constexpr (OUT_BF16) ((uint16_t*)p.out)[oo] = (uint16_t)f2bf16(v);
    else ((float*)p.out)[oo] = v;
    if (p.lse != nullptr && d == 0)
      p.lse[pq] = Wt > 0.f ? (M + log2f(Wt)) * 0.69314718055994531f : -INFINITY;
  }
}

// ---------------------------------------------------------------- dispatch
hipError_t launch_decode_split(int D, int C, int bits, bool qf32, const DecodeParams& p, int grid,
                               hipStream_t s) {
#define LVQ_CASE(d, c, b) if (D == d && C == c && bits == b) return launch_split_t<d, c, b, false, false>(p, qf32, grid, s);
  LVQ_CASE(128, 4, 8) LVQ_CASE(128, 8, 8) LVQ_CASE(128, 2, 8)
  LVQ_CASE(128, 4, 4) LVQ_CASE(128, 8, 4) LVQ_CASE(128, 2, 4)
  LVQ_CASE(64, 2, 4) LVQ_CASE(64, 4, 4) LVQ_CASE(64, 2, 8) LVQ_CASE(64, 4, 8) LVQ_CASE(64, 8, 8)
#undef LVQ_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(int D, bool out_bf16, const CombineParams& p, hipStream_t s) {
  const int grid = p.B * p.H_q;
  if (grid == 0) return hipSuccess;
  if (D == 128) {
    if (out_bf16) hipLaunchKernelGGL((decode_combine_kernel<128, true>), dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_combine_kernel<128, false>), dim3(grid), dim3(256), 0, s, p);
  } else {
    if (out_bf16) hipLaunchKernelGGL((decode_combine_kernel<64, true>), dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_combine_kernel<64, false>), dim3(grid), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace loopvq
