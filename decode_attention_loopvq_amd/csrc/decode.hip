// Combine kernel and the split-kernel launchers (shared codebooks).  The
// split kernel itself is in decode_split.h.
#include "decode_split.h"

namespace loopvq {

// ---- combine: one wave per (request, query head), D/64 channels per lane.
//      The partials are the chunks of the coded positions and, when given, one
//      partial over the request's bf16 tokens (sink and recent window); all are
//      merged by their log-sum-exp.  Chunks go in batches of 16 whose lse and
//      output loads are issued together (one memory round trip per batch);
//      the running maximum rescales the sums when a batch raises it.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(64) void decode_combine_kernel(CombineParams p) {
  constexpr int CPL = D / 64;            // channels per lane
  constexpr int NB = 16;                 // chunks per batch
  const int pq = blockIdx.x;
  const int b = pq / p.H_q, jq = pq - b * p.H_q;
  const int h = jq / p.grp, k = b * p.grp + (jq - h * p.grp);
  const size_t base = (size_t)(h * p.n_pairs + k) * p.n_chunks;
  const size_t wpart = (size_t)h * p.n_pairs + k;
  const int c0l = (int)threadIdx.x * CPL;    // the lane's first channel
  // a batch's loads depend on the plan's chunk count only (indices clamped
  // into it, no branches), so the first batch goes out together with the
  // seq_lens read instead of after it; chunks at or past the request's own
  // count are dropped once that count is known
  // (lane i of the first NB reads the lse of chunk cb + i: a vector load,
  // which goes out with the value loads; scalar loads would wait behind the
  // seq_lens read)
  float lel, le[NB], o[NB][CPL];
  auto load_batch = [&](int cb) {
    lel = p.part_lse[base + min(cb + ((int)threadIdx.x & (NB - 1)), p.n_chunks - 1)];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float* op = p.part_o + (base + min(cb + i, p.n_chunks - 1)) * D + c0l;
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[i][c] = op[c];
    }
  };
  load_batch(0);
  const int len = min(max(p.seq_lens[b], 0), p.max_seq_len);
  const int npart = len > 0 ? (len + p.Lc - 1) / p.Lc : 0;
  float M = -INFINITY, W = 0.f, acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  // the bf16-token partial opens the running sums
  if (p.win_lse != nullptr) {
    const float wle = p.win_lse[wpart];
    if (wle != -INFINITY) {
      M = wle;
      W = 1.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = p.win_o[wpart * D + c0l + c];
    }
  }
  for (int cb = 0; cb < npart; cb += NB) {
    if (cb > 0) load_batch(cb);
    // chunks past the request's end hold stale values: weight 0, value 0
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const bool ok = cb + i < npart;
      le[i] = ok ? u2f(__builtin_amdgcn_readlane(f2u(lel), i)) : -INFINITY;
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[i][c] = ok ? o[i][c] : 0.f;
    }
    float mb = M;
#pragma unroll
    for (int i = 0; i < NB; ++i) mb = fmaxf(mb, le[i]);
    if (mb == -INFINITY) continue;       // nothing yet: every weight is zero
    // exp2(-inf) = 0: sums that are still empty stay empty
    const float sc = __builtin_amdgcn_exp2f(M - mb);
    W *= sc;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] *= sc;
    M = mb;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float wt = le[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(le[i] - M);
      W += wt;
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = fmaf(wt, o[i][c], acc[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const float v = W > 0.f ? acc[c] / W : 0.f;
    const size_t oo = (size_t)pq * D + c0l + c;
    if constexpr (OUT_BF16) ((uint16_t*)p.out)[oo] = (uint16_t)f2bf16(v);
    else ((float*)p.out)[oo] = v;
  }
  if (p.lse != nullptr && threadIdx.x == 0)
    p.lse[pq] = W > 0.f ? (M + log2f(W)) * 0.69314718055994531f : -INFINITY;
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
    if (out_bf16) hipLaunchKernelGGL((decode_combine_kernel<128, true>), dim3(grid), dim3(64), 0, s, p);
    else hipLaunchKernelGGL((decode_combine_kernel<128, false>), dim3(grid), dim3(64), 0, s, p);
  } else {
    if (out_bf16) hipLaunchKernelGGL((decode_combine_kernel<64, true>), dim3(grid), dim3(64), 0, s, p);
    else hipLaunchKernelGGL((decode_combine_kernel<64, false>), dim3(grid), dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace loopvq
