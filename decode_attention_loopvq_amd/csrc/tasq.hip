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
// MI355X mapping: one wave per (token, loop step), up to four tokens of one
// step at a time per workgroup, and about four workgroups per CU that walk
// their step's tokens.  The workgroup first inverts the block's pair
// permutation into LDS, once.  The wave reads the token's H*D keys and weights in
// 16-byte runs, sums the weighted squares in fp64 (the sum then matches an
// exact evaluation except within fp64 rounding of an fp16 rounding midpoint)
// and reduces across lanes with shuffles; every lane then holds sigma.  A
// second pass over the same values forms u = w k * (1 / sigma) in fp64,
// rounds it once to fp32 and writes it to its u position in the wave's LDS
// row; the row then goes out in 16-byte runs.  When H*D <= 2048 the passes
// are unrolled: every load of the token is issued at once and the values stay
// in registers for the second pass (larger rows loop and re-read them from
// the caches); the step's weights and the lane's u positions are read once
// per wave, and with bf16 keys the next token's keys load while the current
// one is transformed.  The fp64 arithmetic (half the fp32 rate), not the 6
// bytes per bf16 element of HBM traffic, bounds the pass.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace loopvq {

template <bool XF32>
__device__ __forceinline__ double load_x(const void* x, size_t i) {
  if constexpr (XF32) return (double)((const float*)x)[i];
  else return (double)u2f((uint32_t)((const uint16_t*)x)[i] << 16);
}

template <bool XF32>
__device__ __forceinline__ void load_run(const void* x, size_t off, float* v) {
  if constexpr (XF32) {
    const float4v a = *(const float4v*)((const float*)x + off);
    const float4v b = *(const float4v*)((const float*)x + off + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4v a = *(const uint4v*)((const uint16_t*)x + off);
    const uint32_t wd[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = bf16lo(wd[i]); v[2 * i + 1] = bf16hi(wd[i]); }
  }
}

// NIT > 0: H*D <= 512*NIT, the passes unrolled over registers; NIT = 0: any H*D
template <bool XF32, int NIT>
__global__ __launch_bounds__(256) void tasq_transform_kernel(TasqParams p) {
  extern __shared__ int tsm[];                // [H][D/2] inverse pair permutation, then one u row per wave
  const int s = blockIdx.y;
  const int step = p.first_step + s;
  const int D = p.D, D2 = p.D / 2, HD = p.H * p.D;
  int* tinv = tsm;                            // u pair holding each RoPE frequency
  const int32_t* perm = p.perm + (size_t)(step / p.Tc) * p.H * D2;
  for (int i = threadIdx.x; i < p.H * D2; i += blockDim.x) {
    const int h = i / D2;
    const int f = perm[i];
    if ((unsigned)f < (unsigned)D2) tinv[h * D2 + f] = i - h * D2;   // out-of-range entries are ignored
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* urow = (float*)(tsm + p.H * D2) + (size_t)wave * HD;
  const float* w = p.w + (size_t)step * HD;
  // sigma in fp16 from the sum of (w k)^2 over a token's H*D values (written
  // once per token at its slot); returns 1 / sigma, or 0 when sigma is 0
  auto finish_sigma = [&](double acc, int slot) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    const _Float16 s16 = (_Float16)(float)sqrt(acc / (double)HD);
    if (lane == 0) p.sigma[(size_t)step * p.sigma_stride + slot] = __builtin_bit_cast(uint16_t, s16);
    return (float)s16 > 0.f ? 1.0 / (double)(float)s16 : 0.0;
  };
  // the LDS row, complete, goes out in 16-byte runs
  auto write_row = [&](size_t xoff) {
    __builtin_amdgcn_s_waitcnt(0xc07f);        // lgkmcnt(0): this wave's row is in LDS
    __asm__ __volatile__("" ::: "memory");
    for (int e0 = lane * 8; e0 < HD; e0 += 512) {
      const float4v a = *(const float4v*)(urow + e0), b = *(const float4v*)(urow + e0 + 4);
      float* out = p.u + xoff + e0;
      *(float4v*)out = a;
      *(float4v*)(out + 4) = b;
    }
  };
  // the workgroup walks the step's tokens, one per wave at a time, so the
  // inverse permutation is built once per workgroup
  const int wpb = blockDim.x >> 6;
  const int j0 = blockIdx.x * wpb + wave, js = gridDim.x * wpb;
  if constexpr (NIT > 0) {
    // 8 consecutive values per lane and pass.  The step's weights and the u
    // position of each of the lane's values are the same for every token, so
    // they are read once; with bf16 keys the next token's keys (and slot) are
    // loaded while the current one is transformed
    constexpr int XW = XF32 ? 8 : 4;
    float wv[NIT][8];
    int uo[NIT][8];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int e0 = lane * 8 + it * 512;
      if (e0 < HD) {
        load_run<true>(w, e0, wv[it]);
        const int h = e0 / D, f0 = e0 - h * D;
        const int side = f0 >= D2 ? 1 : 0, fq = f0 - side * D2;   // the 8 channels lie in one half
#pragma unroll
        for (int i = 0; i < 8; ++i) uo[it][i] = h * D + side + 2 * min(max(tinv[h * D2 + fq + i], 0), D2 - 1);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) { wv[it][i] = 0.f; uo[it][i] = 0; }
      }
    }
    struct Tok { uint32_t x[NIT][XW]; int slot; };
    auto load_tok = [&](int j, Tok& t) {
      const size_t xoff = ((size_t)s * p.n_tok + j) * HD;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int e0 = lane * 8 + it * 512;
        if (e0 < HD) {
          if constexpr (XF32) {
            const uint4v a = *(const uint4v*)((const float*)p.xk + xoff + e0);
            const uint4v b = *(const uint4v*)((const float*)p.xk + xoff + e0 + 4);
            t.x[it][0] = a.x; t.x[it][1] = a.y; t.x[it][2] = a.z; t.x[it][3] = a.w;
            t.x[it][4] = b.x; t.x[it][5] = b.y; t.x[it][6] = b.z; t.x[it][7] = b.w;
          } else {
            const uint4v a = *(const uint4v*)((const uint16_t*)p.xk + xoff + e0);
            t.x[it][0] = a.x; t.x[it][1] = a.y; t.x[it][2] = a.z; t.x[it][3] = a.w;
          }
        }
      }
      t.slot = p.slot_mapping[j];
    };
    auto do_tok = [&](int j, const Tok& t) {
      auto keys = [&](int it, float* x) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if constexpr (XF32) x[i] = u2f(t.x[it][i]);
          else x[i] = (i & 1) ? bf16hi(t.x[it][i >> 1]) : bf16lo(t.x[it][i >> 1]);
        }
      };
      double acc = 0.0;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        if (lane * 8 + it * 512 < HD) {
          float x[8];
          keys(it, x);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const double y = (double)x[i] * (double)wv[it][i];
            acc = fma(y, y, acc);
          }
        }
      }
      const double inv = finish_sigma(acc, t.slot);
      // u: key channel f of head h (f < D/2 or its partner f + D/2) goes to u
      // channel 2*inv[f] (or 2*inv[f] + 1) of that head, through the LDS row
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        if (lane * 8 + it * 512 < HD) {
          float x[8];
          keys(it, x);
#pragma unroll
          for (int i = 0; i < 8; ++i) urow[uo[it][i]] = (float)((double)x[i] * (double)wv[it][i] * inv);
        }
      }
      write_row(((size_t)s * p.n_tok + j) * HD);
    };
    Tok ta, tb;
    if constexpr (XF32) {
      // fp32 keys take twice the registers: no second token in flight
      for (int j = j0; j < p.n_tok; j += js) {
        load_tok(j, ta);
        do_tok(j, ta);
      }
    } else {
      if (j0 < p.n_tok) load_tok(j0, ta);
      for (int j = j0; j < p.n_tok; j += 2 * js) {
        if (j + js < p.n_tok) load_tok(j + js, tb);
        do_tok(j, ta);
        if (j + js >= p.n_tok) break;
        if (j + 2 * js < p.n_tok) load_tok(j + 2 * js, ta);
        do_tok(j + js, tb);
      }
    }
  } else {
    for (int j = j0; j < p.n_tok; j += js) {
      const size_t xoff = ((size_t)s * p.n_tok + j) * HD;
      // u: key channel f of head h goes to u channel 2*inv[f] (+1 for f + D/2)
      auto put_u = [&](int e0, const float* x, const float* wv, double inv) {
        const int h = e0 / D, f0 = e0 - h * D;
        const int side = f0 >= D2 ? 1 : 0, fq = f0 - side * D2;   // the 8 channels lie in one half
        float* dst = urow + h * D + side;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int pp = min(max(tinv[h * D2 + fq + i], 0), D2 - 1);
          dst[2 * pp] = (float)((double)x[i] * (double)wv[i] * inv);
        }
      };
      double acc = 0.0;
      for (int e0 = lane * 8; e0 < HD; e0 += 512) {
        float x[8], wv[8];
        load_run<XF32>(p.xk, xoff + e0, x);
        load_run<true>(w, e0, wv);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double y = (double)x[i] * (double)wv[i];
          acc = fma(y, y, acc);
        }
      }
      const double inv = finish_sigma(acc, p.slot_mapping[j]);
      for (int e0 = lane * 8; e0 < HD; e0 += 512) {
        float x[8], wv[8];
        load_run<XF32>(p.xk, xoff + e0, x);
        load_run<true>(w, e0, wv);
        put_u(e0, x, wv, inv);
      }
      write_row(xoff);
    }
  }
}

hipError_t launch_tasq_transform(bool xf32, const TasqParams& p, int n_steps, hipStream_t s) {
  if (p.n_tok == 0 || n_steps == 0) return hipSuccess;
  const int HD = p.H * p.D;
  // four tokens per workgroup while their rows fit next to the permutation in 64 KiB
  const int wpb = (size_t)4 * HD * 4 + (size_t)HD * 2 <= 65536 ? 4 : 1;
  // about four resident workgroups per CU over all steps; each walks its
  // step's tokens
  const int per_step = std::max(1, 1024 / n_steps);
  const dim3 grid(std::min((p.n_tok + wpb - 1) / wpb, per_step), n_steps);
  const size_t lds = (size_t)wpb * HD * 4 + (size_t)HD * 2;
#define LVQ_TQ(XF, NI) hipLaunchKernelGGL((tasq_transform_kernel<XF, NI>), grid, dim3(64 * wpb), lds, s, p)
  if (HD <= 1024) {
    if (xf32) LVQ_TQ(true, 2); else LVQ_TQ(false, 2);
  } else if (HD <= 2048) {
    if (xf32) LVQ_TQ(true, 4); else LVQ_TQ(false, 4);
  } else {
    if (xf32) LVQ_TQ(true, 0); else LVQ_TQ(false, 0);
  }
#undef LVQ_TQ
  return hipGetLastError();
}

}  // namespace loopvq
