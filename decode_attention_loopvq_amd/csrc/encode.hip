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

template <int G, int C, bool XF32, int BITS>
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

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
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
  const int UPT = n / 16;              // work units (16 groups each) per token (1, 2 or 4)
  const int LUPT = __builtin_ctz(UPT);
  const int R = n * BITS / 8;
  const int P = 1 << p.log2P;
  const void* xsrc = kv ? p.xv : p.xk;
  constexpr int CH = KSTEP < C ? KSTEP : C;   // elements per contiguous run
  const int u0 = (blockIdx.x * 4 + wave) * p.tok_per_wave * UPT;
  const int u1 = min(u0 + p.tok_per_wave * UPT, p.n_tok * UPT);
  if (u0 >= u1) return;                // no work (no barrier follows)

  // raw operand elements of one unit, loaded as fp32 (exact for bf16 and fp32)
  // KSTEP elements per lane and MFMA: runs of `ch` contiguous channels of one
  // loop step; elements past the reduction length KD are zero
  struct Raw { float v[NMF][KSTEP]; };
  // element offset of run (mu, jc) of this lane: a lane-constant part (loop
  // step, channel) plus a wave-uniform part (token, head, group batch)
  const size_t step_stride = (size_t)p.n_tok * H * D;
  size_t lane_off[NMF][KSTEP / CH];
  bool run_ok[NMF][KSTEP / CH];
#pragma unroll
  for (int mu = 0; mu < NMF; ++mu)
#pragma unroll
    for (int q = 0; q < KSTEP / CH; ++q) {
      const int kap = mu * MF + kc * KSTEP + q * CH;
      run_ok[mu][q] = kap < KD;
      const int kp = (XF32 && kap >= G) ? kap - G : kap;
      const int m = kp / C, i0 = kp - m * C;
      lane_off[mu][q] = (size_t)(beta * Tc + m) * step_stride + (size_t)col * C + i0;
    }
  // row slot of group g (the row order of the cache; q = n/8 is a power of two)
  const int lq = __builtin_ctz(n >> 3), hgr = n >> 1;
  auto slot_of = [&](int g) {
    const bool hi = g >= hgr;
    const int gg = hi ? g - hgr : g;
    return ((gg >> lq) << (lq + 1)) + (hi ? (1 << lq) : 0) + (gg & ((1 << lq) - 1));
  };
  auto load_raw = [&](int u, Raw& r) {
    const int uu = min(u, u1 - 1);                 // clamped: loads stay in bounds
    const int tok = uu >> LUPT, gb = uu & (UPT - 1);
    const size_t uoff = ((size_t)tok * H + h) * D + (size_t)gb * 16 * C;
#pragma unroll
    for (int mu = 0; mu < NMF; ++mu)
#pragma unroll
      for (int q = 0; q < KSTEP / CH; ++q) {
        float v[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) v[j] = 0.f;
        if (run_ok[mu][q]) load_run<XF32, CH>(xsrc, uoff + lane_off[mu][q], v);
#pragma unroll
        for (int j = 0; j < CH; ++j) r.v[mu][q * CH + j] = v[j];
      }
  };
  // fp16 operand: bf16 values convert exactly; fp32 values are split into a
  // high part (reduction index < G) and a low part (index >= G)
  auto to_operand = [&](const Raw& r, OpT* Bv) {
#pragma unroll
    for (int mu = 0; mu < NMF; ++mu) {
#pragma unroll
      for (int j = 0; j < KSTEP; ++j) {
        const int kap = mu * MF + kc * KSTEP + j;
        const float v = r.v[mu][j];
        const _Float16 hi = (_Float16)v;
        Bv[mu][j] = (XF32 && kap >= G && kap < KD) ? (_Float16)(v - (float)hi) : hi;
      }
    }
  };

  // software pipeline over units: the raw loads of unit u+3 are issued while
  // unit u is scored
  Raw rb[4];
  load_raw(u0, rb[0]);
  load_raw(u0 + 1, rb[1]);
  load_raw(u0 + 2, rb[2]);
  auto do_unit = [&](int u, Raw& cur, Raw& nxt) {
    OpT Bv[NMF];
    to_operand(cur, Bv);
    load_raw(u + 3, nxt);
    const int tok = u >> LUPT, gb = u & (UPT - 1);
    const int slot = p.slot_mapping[tok];
    // ---- scores against all entries: per 16-entry tile the lane sees 4
    //      entries (rows 4*kc .. 4*kc+3) of its vector.  It keeps the best
    //      tile (strict compare in increasing tile order) and that tile's four
    //      scores; the lowest row holding the maximum is resolved at the end,
    //      so the whole search takes the lowest index on exact ties.
    float best = -INFINITY, bd0 = 0.f, bd1 = 0.f, bd2 = 0.f, bd3 = 0.f;
    int btile = 0;
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      float4v d = Cin[t];
#pragma unroll
      for (int mu = 0; mu < NMF; ++mu) {
        if constexpr (MF == 32) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[t][mu], Bv[mu], d, 0, 0, 0);
        else d = __builtin_amdgcn_mfma_f32_16x16x16f16(A[t][mu], Bv[mu], d, 0, 0, 0);
      }
      float m3 = __builtin_fmaxf(__builtin_fmaxf(d.x, d.y), d.z);
      m3 = __builtin_fmaxf(m3, d.w);
      const bool better = m3 > best;
      best = better ? m3 : best;
      btile = better ? t : btile;
      bd0 = better ? d.x : bd0;
      bd1 = better ? d.y : bd1;
      bd2 = better ? d.z : bd2;
      bd3 = better ? d.w : bd3;
    }
    const int r = bd0 == best ? 0 : (bd1 == best ? 1 : (bd2 == best ? 2 : 3));
    int bidx = 16 * btile + 4 * kc + r;
    // ---- merge the four lanes holding the same vector (lower index on ties)
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float ob = __shfl_xor(best, off);
      const int oi = __shfl_xor(bidx, off);
      const bool take = ob > best || (ob == best && oi < bidx);
      best = take ? ob : best;
      bidx = take ? oi : bidx;
    }
    // ---- write the code into its row slot
    uint8_t* row = p.cache + (int64_t)beta * p.block_stride +
                   ((((size_t)(slot >> p.log2P) * H + h) * 2 + kv) * P + (slot & (P - 1))) * R;
    const int sl = slot_of(gb * 16 + col);
    if constexpr (BITS == 8) {
      if (kc == 0) row[sl] = (uint8_t)bidx;
    } else {
      const int other = __shfl_xor(bidx, 1);
      if (kc == 0 && (col & 1) == 0) row[sl >> 1] = (uint8_t)((bidx & 15) | ((other & 15) << 4));
    }
  };
  int u = u0;
  for (; u + 4 <= u1; u += 4) {
    do_unit(u, rb[0], rb[3]);
    do_unit(u + 1, rb[1], rb[0]);
    do_unit(u + 2, rb[2], rb[1]);
    do_unit(u + 3, rb[3], rb[2]);
  }
  if (u < u1) do_unit(u, rb[0], rb[3]);
  if (u + 1 < u1) do_unit(u + 1, rb[1], rb[0]);
  if (u + 2 < u1) do_unit(u + 2, rb[2], rb[1]);
}

template <int G, int C, bool XF32, int BITS>
static hipError_t launch_encode_t(const EncodeParams& p, int n_blocks, hipStream_t s) {
  dim3 grid(p.n_tok_groups, n_blocks * 2 * p.H_kv);
  hipLaunchKernelGGL((encode_kernel<G, C, XF32, BITS>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_encode(int G, bool xf32, int bits, const EncodeParams& p, int n_blocks, hipStream_t s) {
  const int c = p.c;
#define LVQ_ENC(g, cc, f, b) \
  if (G == g && c == cc && xf32 == f && bits == b) return launch_encode_t<g, cc, f, b>(p, n_blocks, s);
#define LVQ_ENC_C(g, f, b) LVQ_ENC(g, 2, f, b) LVQ_ENC(g, 4, f, b) LVQ_ENC(g, 8, f, b)
  LVQ_ENC_C(16, false, 8) LVQ_ENC_C(32, false, 8) LVQ_ENC_C(16, false, 4) LVQ_ENC_C(32, false, 4)
  LVQ_ENC_C(8, true, 8) LVQ_ENC_C(16, true, 8) LVQ_ENC_C(32, true, 8)
  LVQ_ENC_C(8, true, 4) LVQ_ENC_C(16, true, 4) LVQ_ENC_C(32, true, 4)
#undef LVQ_ENC_C
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
