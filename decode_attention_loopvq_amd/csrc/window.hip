// Decode attention over the bf16 tokens of each request: the attention sink
// and the recent window.
//
// What it computes [LoopVQ paper, hub.valency.io/works/W_7srt5hed_v1,
// section "System implementation", cache layout and attention]: a request's
// leading n_s tokens and its latest tokens live unquantised in bf16 pages of
// 8 tokens and every other token as codes; each loop step attends the two
// kinds of page in separate kernels and joins their partial outputs by
// log-sum-exp.  This kernel is the bf16 side: it leaves one
// partial (o, log2-sum-exp) per (request, query head) for the combine kernel.
// The bf16 pages hold pre-RoPE keys (they are coded later, when the window
// moves on), so the key is rotated here at its token's position, with the
// same RoPE table as the coded side.
//
// MI355X mapping: one workgroup of four waves per (request, query head).  A
// wave takes 16 tokens per step; lane (slot ts, quarter cq) owns token ts and
// the quarter cq of the RoPE frequencies (channels cq*F .. cq*F+F-1 and
// their partners D/2 + ...), so each lane reads two contiguous 2F-byte runs of
// K and of V.  The quarter sums meet through two lane swaps; each lane then
// keeps its own online softmax over its tokens, and the workgroup merges the
// 256 lane states through LDS at the end.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace loopvq {

template <int D, bool QF32>
__global__ __launch_bounds__(256) void decode_window_kernel(WindowParams p) {
  constexpr int F = D / 8;              // frequencies per lane quarter
  constexpr int FP = F / 2;             // float4 table words per quarter
  constexpr int NW = 4;                 // waves
  constexpr int RS = 2 * F + 1;         // padded floats per lane state in LDS
  __shared__ float red_acc[NW * 64 * RS];
  __shared__ float red_m[NW * 64];
  __shared__ float red_l[NW * 64];

  const int pq = blockIdx.x;
  const int b = pq / p.H_q, jq = pq - b * p.H_q;
  const int h = jq / p.grp, k = b * p.grp + (jq - h * p.grp);
  const int len = min(max(p.seq_lens[b], 0), p.max_seq_len);
  const int ns = min(max(p.n_sink[b], 0), len);
  const int ws = min(max(p.win_start[b], ns), len);
  const int nbf = ns + (len - ws);      // bf16 tokens: u < ns at position u, then ws + (u - ns)

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int ts = lane >> 2, cq = lane & 3;

  // query quarter: q_f and q_h of the lane's frequencies
  float qf[F], qh[F];
  {
    const size_t qo = ((size_t)b * p.H_q + jq) * D + cq * F;
#pragma unroll
    for (int i = 0; i < F; ++i) {
      if constexpr (QF32) {
        qf[i] = ((const float*)p.q)[qo + i];
        qh[i] = ((const float*)p.q)[qo + D / 2 + i];
      } else {
        qf[i] = u2f((uint32_t)((const uint16_t*)p.q)[qo + i] << 16);
        qh[i] = u2f((uint32_t)((const uint16_t*)p.q)[qo + D / 2 + i] << 16);
      }
    }
  }

  float m = -INFINITY, l = 0.f;
  float acc[2 * F];
#pragma unroll
  for (int i = 0; i < 2 * F; ++i) acc[i] = 0.f;

  const int32_t* pt = p.page_table + (size_t)b * p.max_pages;
  for (int u0 = wave * 16; u0 < nbf; u0 += NW * 16) {
    const int u = u0 + ts;
    const bool valid = u < nbf;
    const int uu = min(u, nbf - 1);
    const int pos = uu < ns ? uu : ws + (uu - ns);
    const int page = pt[min(uu >> 3, p.max_pages - 1)];
    const uint16_t* krow = p.kv + (((size_t)page * p.H_kv + h) * 2 * 8 + (uu & 7)) * D + cq * F;
    const uint16_t* vrow = krow + 8 * D;
    // K and V runs of the lane's channels, bf16 pairs
    uint4v kr[F / 4], vr[F / 4];
#pragma unroll
    for (int j = 0; j < F / 8; ++j) {
      kr[j] = *(const uint4v*)(krow + 8 * j);
      kr[F / 8 + j] = *(const uint4v*)(krow + D / 2 + 8 * j);
      vr[j] = *(const uint4v*)(vrow + 8 * j);
      vr[F / 8 + j] = *(const uint4v*)(vrow + D / 2 + 8 * j);
    }
    const float4v* tr = (const float4v*)p.rope + (size_t)(pos >> 2) * FP * 16 + cq * 4 + (pos & 3);
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int j = 0; j < FP; ++j) {
      const float4v cs = tr[j * 16];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 2 * j + e;
        const uint32_t wf = ((const uint32_t*)&kr[i / 8])[(i % 8) / 2];
        const uint32_t wh = ((const uint32_t*)&kr[F / 8 + i / 8])[(i % 8) / 2];
        const float kf = (i & 1) ? bf16hi(wf) : bf16lo(wf);
        const float kh = (i & 1) ? bf16hi(wh) : bf16lo(wh);
        // q . RoPE(k) for this frequency: cos*(qf kf + qh kh) + sin*(qh kf - qf kh)
        const float X = fmaf(qh[i], kh, qf[i] * kf);
        const float Y = fmaf(-qf[i], kh, qh[i] * kf);
        sa = fmaf(e ? cs.z : cs.x, X, sa);
        sb = fmaf(e ? cs.w : cs.y, Y, sb);
      }
    }
    float sc = sa + sb;
    sc += __shfl_xor(sc, 1);
    sc += __shfl_xor(sc, 2);
    const float s = valid ? sc * p.scale_log2 : -INFINITY;
    if (s > m) {
      const float f = __builtin_amdgcn_exp2f(m - s);   // 0 when m = -inf
      l *= f;
#pragma unroll
      for (int i = 0; i < 2 * F; ++i) acc[i] *= f;
      m = s;
    }
    const float pv = valid ? __builtin_amdgcn_exp2f(s - m) : 0.f;
    l += pv;
#pragma unroll
    for (int i = 0; i < F; ++i) {
      const uint32_t wf = ((const uint32_t*)&vr[i / 8])[(i % 8) / 2];
      const uint32_t wh = ((const uint32_t*)&vr[F / 8 + i / 8])[(i % 8) / 2];
      acc[i] = fmaf(pv, (i & 1) ? bf16hi(wf) : bf16lo(wf), acc[i]);
      acc[F + i] = fmaf(pv, (i & 1) ? bf16hi(wh) : bf16lo(wh), acc[F + i]);
    }
  }

  // ---- merge the 256 lane states: common maximum, then per-channel sums
  red_m[tid] = m;
  __syncthreads();
  float M = -INFINITY;
  for (int i = 0; i < NW * 64; ++i) M = fmaxf(M, red_m[i]);
  const float sc = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
#pragma unroll
  for (int i = 0; i < 2 * F; ++i) red_acc[tid * RS + i] = acc[i] * sc;
  red_l[tid] = l * sc;
  __syncthreads();
  const size_t part = (size_t)h * p.n_pairs + k;
  if (tid < D) {
    const int dcq = (tid % (D / 2)) / F;
    const int di = (tid >= D / 2 ? F : 0) + (tid % (D / 2)) % F;
    float o = 0.f, L = 0.f;
    for (int w = 0; w < NW; ++w)
      for (int t2 = 0; t2 < 16; ++t2) {
        const int src = w * 64 + t2 * 4 + dcq;
        o += red_acc[src * RS + di];
        L += red_l[src];      // each token's p counted once per quarter: sum one quarter's lanes
      }
    p.win_o[part * D + tid] = L > 0.f ? o / L : 0.f;
    if (tid == 0) p.win_lse[part] = L > 0.f ? M + log2f(L) : -INFINITY;
  }
}

hipError_t launch_decode_window(int D, bool qf32, const WindowParams& p, int B, hipStream_t s) {
  const int grid = B * p.H_q;
  if (grid == 0) return hipSuccess;
  if (D == 128) {
    if (qf32) hipLaunchKernelGGL((decode_window_kernel<128, true>), dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_window_kernel<128, false>), dim3(grid), dim3(256), 0, s, p);
  } else {
    if (qf32) hipLaunchKernelGGL((decode_window_kernel<64, true>), dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_window_kernel<64, false>), dim3(grid), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace loopvq
