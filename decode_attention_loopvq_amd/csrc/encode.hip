// LoopVQ encoder on gfx950: nearest codebook entry of every coupled vector.
//
// What it computes [LoopVQ paper, hub.valency.io/works/W_7srt5hed_v1,
// section "Loop-axis vector quantization", eq. (4), and section
// "Preliminaries", eq. (2); section "System implementation",
// encoding]: for token j, KV head h, x in {K, V}, block beta and group g the
// coupled vector z[i*Tc + m] = x^(beta*Tc+m+1)[j][h][g*c + i] is replaced by
// argmin_r ||z - e_r||^2 (lowest r on ties), written into the paged index row.
//
// MI355X mapping:
//  * argmin ||z - e||^2 = argmax (z.e - 0.5*||e||^2): the dot products are one
//    fp16 MFMA per 16 entries x 16 vectors, with -0.5*||e||^2 loaded as the
//    accumulator input, so the distance needs no VALU work beyond the argmax.
//  * The MFMA reduction index runs over the coupled coordinates in loop-major
//    order (kappa = m*c + i) on both operands, so a lane's operand is c
//    contiguous channels of one loop step (one 8- or 16-byte load).  bf16
//    inputs convert to fp16 exactly inside fp16's normal range; fp32 inputs
//    are split into an fp16 high and low part placed side by side along the
//    reduction index (against two copies of the entry).
//  * Rows of the MFMA are codebook entries, columns are vectors: a lane sees 4
//    entries of one vector per MFMA and keeps a running (best, index) with a
//    strict compare in increasing entry order (lowest index on ties); the four
//    lanes that share a vector merge at the end with a lexicographic compare.
//  * The whole codebook tile set stays in registers for the life of the wave.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace loopvq {

template <bool XF32, int CH>
__device__ __forceinline__ void load_run(const void* base, size_t off, float* v) {
  if constexpr (XF32) {
    const float* s = (const float*)base + off;
#pragma unroll
    for (int j = 0; j < CH; ++j) v[j] = s[j];
  } else {
    const uint16_t* s = (const uint16_t*)base + off;
    if constexpr (CH == 8) {
      uint4v w = *(const uint4v*)s;
      uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) { v[2 * j] = bf16lo(ww[j]); v[2 * j + 1] = bf16hi(ww[j]); }
    } else if constexpr (CH == 4) {
      uint2v w = *(const uint2v*)s;
      v[0] = bf16lo(w.x); v[1] = bf16hi(w.x); v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
    } else if constexpr (CH == 2) {
      uint32_t w = *(const uint32_t*)s;
      v[0] = bf16lo(w); v[1] = bf16hi(w);
    } else {
#pragma unroll
      for (int j = 0; j < CH; ++j) v[j] = u2f((uint32_t)s[j] << 16);
    }
  }
}

template <int G, bool XF32, int BITS>
__global__ __launch_bounds__(256) void encode_kernel(EncodeParams p) {
  constexpr int KD = XF32 ? 2 * G : G;          // reduction length with the fp32 split
  constexpr int KDP = KD < 16 ? 16 : KD;        // padded to the MFMA depth
  constexpr int MF = (KDP % 32 == 0) ? 32 : 16; // 16x16x32 or 16x16x16
  constexpr int KSTEP = MF / 4;                 // operand elements per lane per MFMA
  constexpr int NMF = KDP / MF;
  constexpr int KENT = 1 << BITS;
  constexpr int NTILE = KENT / 16;
  using OpT = typename std::conditional<MF == 32, half8v, half4v>::type;

  __shared__ uint16_t cbp[KENT * G];

  const int H = p.H_kv, c = p.c, Tc = p.Tc, D = p.D;
  const int y = blockIdx.y;
  const int h = y % H, kv = (y / H) & 1, beta = y / (2 * H);

  // ---- codebook of (beta, h, kv), permuted to loop-major coordinates
  const uint16_t* cbsrc = p.cb + ((size_t)(beta * H + h) * 2 + kv) * KENT * G;
  for (int x = threadIdx.x; x < KENT * G; x += blockDim.x) {
    const int e = x / G, kap = x - e * G;
    const int m = kap / c, i = kap - m * c;
    cbp[x] = cbsrc[(size_t)e * G + i * Tc + m];
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kc = lane >> 4, col = lane & 15;

  // ---- entry operands (rows = entries) and -0.5||e||^2 accumulator inputs
  OpT A[NTILE][NMF];
  float4v Cin[NTILE];
  const float* hs = p.hsq + ((size_t)(beta * H + h) * 2 + kv) * KENT;
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
#pragma unroll
    for (int mu = 0; mu < NMF; ++mu) {
#pragma unroll
      for (int j = 0; j < KSTEP; ++j) {
        const int kap = mu * MF + kc * KSTEP + j;
        const uint16_t bits = kap < KD ? cbp[(16 * t + col) * G + (kap % G)] : (uint16_t)0;
        A[t][mu][j] = __builtin_bit_cast(_Float16, bits);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) Cin[t][r] = -hs[16 * t + 4 * kc + r];
  }

  const int n = D / c;                 // groups per token
  const int R = n * BITS / 8;
  const int P = 1 << p.log2P;
  const void* xsrc = kv ? p.xv : p.xk;
  constexpr int CHMAX = KSTEP;
  const int tok0 = (blockIdx.x * 4 + wave) * p.tok_per_wave;
  const int tok1 = min(tok0 + p.tok_per_wave, p.n_tok);

  for (int tok = tok0; tok < tok1; ++tok) {
    const int slot = p.slot_mapping[tok];
    uint8_t* row = p.cache + (int64_t)beta * p.block_stride +
                   ((((size_t)(slot >> p.log2P) * H + h) * 2 + kv) * P + (slot & (P - 1))) * R;
    for (int g0 = 0; g0 < n; g0 += 16) {
      const int g = g0 + col;
      // ---- vector operand (columns = vectors)
      OpT Bv[NMF];
#pragma unroll
      for (int mu = 0; mu < NMF; ++mu) {
        const int k0 = mu * MF + kc * KSTEP;
        // runs of CH contiguous channels of one loop step
        const int CH = KSTEP < c ? KSTEP : c;
#pragma unroll
        for (int j = 0; j < KSTEP; ++j) Bv[mu][j] = (_Float16)0.f;
        for (int jc = 0; jc < KSTEP; jc += CH) {
          const int kap = k0 + jc;
          if (kap >= KD) break;
          const bool lo_part = XF32 && kap >= G;
          const int kp = lo_part ? kap - G : kap;
          const int m = kp / c, i0 = kp - m * c;
          const size_t off = (((size_t)(beta * Tc + m) * p.n_tok + tok) * H + h) * D + g * c + i0;
          float v[CHMAX];
          if (CH == KSTEP) load_run<XF32, KSTEP>(xsrc, off, v);
          else {
#pragma unroll
            for (int j = 0; j < CHMAX; ++j) v[j] = 0.f;
            for (int j = 0; j < CH; ++j) {
              float tmp[1];
              load_run<XF32, 1>(xsrc, off + j, tmp);
              v[j] = tmp[0];
            }
          }
          for (int j = 0; j < CH; ++j) {
            const _Float16 hi = (_Float16)v[j];
            Bv[mu][jc + j] = lo_part ? (_Float16)(v[j] - (float)hi) : hi;
          }
        }
      }
      // ---- scores against all entries, running argmax
      float best = -INFINITY;
      int bidx = 0;
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        float4v d = Cin[t];
#pragma unroll
        for (int mu = 0; mu < NMF; ++mu) {
          if constexpr (MF == 32) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[t][mu], Bv[mu], d, 0, 0, 0);
          else d = __builtin_amdgcn_mfma_f32_16x16x16f16(A[t][mu], Bv[mu], d, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool better = d[r] > best;
          best = better ? d[r] : best;
          bidx = better ? 16 * t + 4 * kc + r : bidx;
        }
      }
      // ---- merge the four lanes holding the same vector
#pragma unroll
      for (int off = 16; off <= 32; off <<= 1) {
        const float ob = __shfl_xor(best, off);
        const int oi = __shfl_xor(bidx, off);
        const bool take = ob > best || (ob == best && oi < bidx);
        best = take ? ob : best;
        bidx = take ? oi : bidx;
      }
      // ---- write the code into its row slot
      const int s = row_slot_of_group(g, n);
      if constexpr (BITS == 8) {
        if (kc == 0) row[s] = (uint8_t)bidx;
      } else {
        const int other = __shfl_xor(bidx, 1);
        if (kc == 0 && (col & 1) == 0) row[s >> 1] = (uint8_t)((bidx & 15) | ((other & 15) << 4));
      }
    }
  }
}

template <int G, bool XF32, int BITS>
static hipError_t launch_encode_t(const EncodeParams& p, int n_blocks, hipStream_t s) {
  dim3 grid(p.n_tok_groups, n_blocks * 2 * p.H_kv);
  hipLaunchKernelGGL((encode_kernel<G, XF32, BITS>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_encode(int G, bool xf32, int bits, const EncodeParams& p, int n_blocks, hipStream_t s) {
#define LVQ_ENC(g, f, b) if (G == g && xf32 == f && bits == b) return launch_encode_t<g, f, b>(p, n_blocks, s);
  LVQ_ENC(16, false, 8) LVQ_ENC(32, false, 8) LVQ_ENC(8, false, 8)
  LVQ_ENC(16, true, 8) LVQ_ENC(8, true, 8) LVQ_ENC(32, true, 8)
  LVQ_ENC(16, false, 4) LVQ_ENC(32, false, 4) LVQ_ENC(8, false, 4)
  LVQ_ENC(16, true, 4) LVQ_ENC(8, true, 4) LVQ_ENC(32, true, 4)
#undef LVQ_ENC
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- load-time slices
// slices[t][h][kv][e][i] = cb[t / Tc][h][kv][e][i*Tc + t % Tc]; hsq = 0.5*||e||^2 (fp64 sum)
__global__ void build_slices_kernel(const uint16_t* __restrict__ cb, uint16_t* __restrict__ slices,
                                    float* __restrict__ hsq, int n_blocks, int H, int K, int c, int Tc) {
  const int G = c * Tc;
  const size_t n_entries = (size_t)n_blocks * H * 2 * K;
  for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < n_entries; x += (size_t)gridDim.x * blockDim.x) {
    const uint16_t* e = cb + x * G;
    // x = ((beta*H + h)*2 + kv)*K + r
    const size_t r = x % K, hk = (x / K) % (2 * (size_t)H), beta = x / (K * 2 * (size_t)H);
    double s = 0.0;
    for (int u = 0; u < G; ++u) {
      const double v = (double)__builtin_bit_cast(_Float16, e[u]);
      s += v * v;
    }
    if (hsq != nullptr) hsq[x] = (float)(0.5 * s);
    for (int m = 0; m < Tc; ++m) {
      uint16_t* dst = slices + ((((size_t)(beta * Tc + m) * 2 * H + hk) * K) + r) * c;
      for (int i = 0; i < c; ++i) dst[i] = e[i * Tc + m];
    }
  }
}

hipError_t launch_build_slices(const uint16_t* cb, uint16_t* slices, float* hsq, int n_blocks, int H_kv,
                               int K, int c, int Tc, hipStream_t s) {
  const size_t n = (size_t)n_blocks * H_kv * 2 * K;
  const int grid = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(build_slices_kernel, dim3(grid > 0 ? grid : 1), dim3(256), 0, s, cb, slices, hsq, n_blocks,
                     H_kv, K, c, Tc);
  return hipGetLastError();
}

}  // namespace loopvq
