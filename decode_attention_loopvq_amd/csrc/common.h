// Shared device/host helpers of the LoopVQ HIP library (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "loopvq.h"

namespace loopvq {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t uint2v __attribute__((ext_vector_type(2)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bit casts
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

// bf16 stored in the low / high half of a 32-bit word -> fp32 (exact)
__device__ __forceinline__ float bf16lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return u2f(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite)
__device__ __forceinline__ uint32_t f2bf16(float f) {
  uint32_t u = f2u(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// two fp32 -> packed fp16 pair (round to nearest even), lo in bits 0..15
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  half2v h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ half2v as_h2(uint32_t w) { return __builtin_bit_cast(half2v, w); }

// fp32 = a.lo*b.lo + a.hi*b.hi + acc, fp16 products exact, fp32 accumulate
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), acc, false);
}
// v_perm_b32: byte n of the result is byte sel.byte[n] of {src0:src1}
// (bytes 0..3 come from src1, 4..7 from src0, 0x0c gives 0x00).
__device__ __forceinline__ uint32_t perm(uint32_t src0, uint32_t src1, uint32_t sel) {
  return __builtin_amdgcn_perm(src0, src1, sel);
}

// DPP row-local lane moves inside groups of four lanes
template <int PAT>
__device__ __forceinline__ float quad_mov(float v) {
  return u2f(__builtin_amdgcn_mov_dpp(f2u(v), PAT, 0xf, 0xf, true));
}
// quad_perm encodings: lane i of each quad reads lane sel_i
constexpr int QP_XOR1 = (1 << 0) | (0 << 2) | (3 << 4) | (2 << 6);   // [1,0,3,2]
constexpr int QP_XOR2 = (2 << 0) | (3 << 2) | (0 << 4) | (1 << 6);   // [2,3,0,1]

__device__ __forceinline__ float quad_sum(float v) {
  v += quad_mov<QP_XOR1>(v);
  v += quad_mov<QP_XOR2>(v);
  return v;
}

// ---------------------------------------------------------------- row order
// Slot s of an index row holds group g(s) ("RoPE-pair interleaved" order):
// n groups, h = n/2, q = n/8; s = i*2q + r; g = i*q + r (r < q) or
// h + i*q + (r - q).  Inverse: slot of group g.
__host__ __device__ __forceinline__ int row_group_of_slot(int s, int n) {
  int q = n >> 3, i = s / (2 * q), r = s % (2 * q);
  return r < q ? i * q + r : (n >> 1) + i * q + (r - q);
}
__host__ __device__ __forceinline__ int row_slot_of_group(int g, int n) {
  int h = n >> 1, q = n >> 3;
  int hi = g >= h, gg = hi ? g - h : g;
  int i = gg / q, r = gg % q;
  return i * 2 * q + (hi ? q + r : r);
}

}  // namespace loopvq
