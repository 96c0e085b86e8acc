// Quantised split-K decode attention for LoopVQ on gfx950.
//
// What it computes [LoopVQ paper, hub.valency.io/works/W_7srt5hed_v1,
// section 4 "System implementation", attention; App. C]: at loop step t every
// cached token j of a request contributes its key rebuilt from the step's
// codebook slice, rotated by RoPE at position j, and its value rebuilt the
// same way; tokens are cut into splits whose partial softmax outputs are
// merged by their logsumexp (combine kernel below), which recovers the exact
// softmax over all tokens.
//
// MI355X mapping (this file's own design, not the pages'):
//  * A wave is 16 "lane blocks" of 4 lanes.  A block is one (request, query
//    head) pair at one position; its 4 lanes each own a quarter of the RoPE
//    frequencies, i.e. D/8 channel pairs {f, f + D/2}.  Blocks of one wave are
//    NP pairs x NT positions (NP*NT = 16), so NP pairs at the same position
//    read the same RoPE-table row (the pages' "several requests per block"
//    table sharing, taken to 16 pairs).
//  * The two index rows of a token are streamed with one load per lane: the
//    cache row order puts the groups a lane needs side by side.
//  * The K and V slices of the workgroup's KV head are staged once in LDS,
//    replicated so that lane l always reads its own bank window: entry e for
//    lane slot s lives at e*256 + kv*128 + s*entry_bytes, so random gathers of
//    one wave hit disjoint banks.  Gather addresses come from one v_perm_b32.
//  * Scores are exact: fp16 codebook channels and fp16 query pairs feed
//    v_dot2_f32_f16 (products exact in fp32), and the fp32 cos/sin weights are
//    applied with fp32 FMAs:  s = sum_f cos_f*X_f + sin_f*Y_f with
//    X_f = q_f k_f + q_{f+D/2} k_{f+D/2} and Y_f = q_{f+D/2} k_f - q_f k_{f+D/2},
//    which equals q . RoPE(k) (rotate-half RoPE).
//  * The value side runs on the matrix cores: v_mfma_f32_4x4x4_16b_f16 with A
//    = p*I (each block is one token, lane i supplies row i) and B = the lane's
//    gathered V entries accumulates p*v in fp32 registers with no VALU work
//    per channel.  p is rounded to fp16 for the product; the running sum l
//    adds the same rounded p, so the output stays an exact convex combination.
//  * Online softmax in the log2 domain with a lazy maximum: the running max m
//    is only raised when a score exceeds it by more than 8 (so p <= 256), which
//    makes rescaling rare.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace loopvq {

constexpr float LAZY_TAU = 8.0f;

template <int LB>
struct RowLoad;
template <> struct RowLoad<1> { static __device__ __forceinline__ void load(const uint8_t* p, uint32_t* w) { w[0] = *p; } };
template <> struct RowLoad<2> { static __device__ __forceinline__ void load(const uint8_t* p, uint32_t* w) { w[0] = *(const uint16_t*)p; } };
template <> struct RowLoad<4> { static __device__ __forceinline__ void load(const uint8_t* p, uint32_t* w) { w[0] = *(const uint32_t*)p; } };
template <> struct RowLoad<8> { static __device__ __forceinline__ void load(const uint8_t* p, uint32_t* w) {
  uint2v v = *(const uint2v*)p; w[0] = v.x; w[1] = v.y; } };
template <> struct RowLoad<16> { static __device__ __forceinline__ void load(const uint8_t* p, uint32_t* w) {
  uint4v v = *(const uint4v*)p; w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w; } };

// LDS address of the entry whose code sits in slot s of the lane's row words
template <int BITS>
__device__ __forceinline__ uint32_t slot_addr(const uint32_t* w, int s, uint32_t lane_off) {
  if constexpr (BITS == 8) {
    // byte 1 <- code, byte 0 <- lane offset, bytes 2,3 <- 0
    return perm(w[s >> 2], lane_off, 0x0c0c0000u | ((4u + (s & 3)) << 8));
  } else {
    uint32_t code = (w[s >> 3] >> ((s & 7) * 4)) & 15u;
    return (code << 8) | lane_off;
  }
}

template <int EB>
struct Entry { uint32_t d[EB / 4]; };

template <int EB>
__device__ __forceinline__ Entry<EB> lds_entry(const uint8_t* lds, uint32_t addr) {
  Entry<EB> e;
  if constexpr (EB == 4) {
    e.d[0] = *(const uint32_t*)(lds + addr);
  } else if constexpr (EB == 8) {
    uint2v v = *(const uint2v*)(lds + addr); e.d[0] = v.x; e.d[1] = v.y;
  } else {
    uint4v v = *(const uint4v*)(lds + addr); e.d[0] = v.x; e.d[1] = v.y; e.d[2] = v.z; e.d[3] = v.w;
  }
  return e;
}

template <int D, int C, int BITS, bool QF32>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeParams p) {
  constexpr int N = D / C;            // groups per row
  constexpr int Q = N / 8;            // lo (and hi) groups per lane quarter
  constexpr int F = D / 8;            // RoPE frequencies per lane quarter
  constexpr int FP = F / 2;           // frequency pairs per quarter (one K MFMA each)
  constexpr int EB = 2 * C;           // bytes of one slice entry
  constexpr int NSLOT = 128 / EB;     // bank windows per 128-byte LDS stripe
  constexpr int R = N * BITS / 8;     // row bytes
  constexpr int LB = R / 4;           // row bytes per lane quarter
  constexpr int LW = (LB + 3) / 4;    // row words per lane
  constexpr int U = D / 16;           // 4-channel V units per lane
  constexpr int KENT = 1 << BITS;
  constexpr int SW = 4 * U + 3;       // floats of one lane's softmax state
  constexpr int LDS_SLICES = KENT * 256;
  constexpr int LDS_MERGE = 4 * 64 * SW * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_SLICES > LDS_MERGE ? LDS_SLICES : LDS_MERGE];

  // ---- workgroup -> (KV head, 4 work items); XCD-contiguous order
  int bid = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int h = bid / p.wg_per_head;
  const int wgi = bid - h * p.wg_per_head;

  // ---- stage the K and V slices of head h, replicated per bank window
  {
    const uint8_t* src = (const uint8_t*)p.slices + (size_t)h * 2 * KENT * EB;
    for (int x = threadIdx.x; x < KENT * 16; x += blockDim.x) {
      const int e = x >> 4, kv = (x >> 3) & 1, cchunk = x & 7;
      const uint8_t* sp = src + ((size_t)kv * KENT + e) * EB;
      uint4v v;
      if constexpr (EB == 16) {
        v = *(const uint4v*)sp;
      } else if constexpr (EB == 8) {
        uint2v t = *(const uint2v*)sp; v = (uint4v){t.x, t.y, t.x, t.y};
      } else {
        uint32_t t = *(const uint32_t*)sp; v = (uint4v){t, t, t, t};
      }
      *(uint4v*)(lds + e * 256 + kv * 128 + cchunk * 16) = v;
    }
  }
  __syncthreads();

  // ---- this wave's work item: (pair group, chunk); lane roles
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int item = wgi * 4 + wave;
  const bool item_ok = item < p.items_per_head;
  const int ch = item_ok ? item / p.n_pg : 0;
  const int pg = item_ok ? item - ch * p.n_pg : 0;
  const int kslot = lane >> 4;               // pair slot of the 16-lane row
  const int la = (lane >> 2) & 3, lb = lane & 3;
  // K role: quarter la, position slot lb.  V role: position slot la, quarter lb.
  const int k = pg * p.NP + kslot % p.NP;
  const int pgrp = kslot / p.NP;             // position group of this row
  const bool pair_ok = item_ok && k < p.n_pairs;
  const int b = pair_ok ? k / p.grp : 0;
  const int jq = h * p.grp + (pair_ok ? k - (k / p.grp) * p.grp : 0);
  const int len = pair_ok ? min(max(p.seq_lens[b], 0), p.max_seq_len) : 0;
  const int p0 = ch * p.Lc;
  const bool active = item_ok && __ballot(p0 < len) != 0;   // wave-uniform

  float m = -INFINITY, l = 0.f, lx = 0.f;   // running max, sum of rounded p, exact sum of p
  float4v acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = (float4v){0.f, 0.f, 0.f, 0.f};

  if (active) {
    // ---- K-side A operands: for frequency pair j, lane lb supplies row lb of
    //      [[q_f, q_h, 0, 0], [q_h, -q_f, 0, 0], [0, 0, q_f', q_h'], [0, 0, q_h', -q_f']]
    //      (f = 2j, f' = 2j+1 of quarter la; q_h = q_{f + D/2}), so the MFMA
    //      yields X_f, Y_f, X_f', Y_f' of the position in each column.
    half4v AK[FP];
    half4v AKl[QF32 ? FP : 1];
    {
      const size_t qoff = ((size_t)b * p.H_q + jq) * D + la * F;
#pragma unroll
      for (int j = 0; j < FP; ++j) {
        const int f = 2 * j + (lb >> 1);     // rows 0,1 use f = 2j, rows 2,3 use 2j+1
        float a, c;
        if constexpr (QF32) {
          a = ((const float*)p.q)[qoff + f];
          c = ((const float*)p.q)[qoff + D / 2 + f];
        } else {
          a = u2f((uint32_t)((const uint16_t*)p.q)[qoff + f] << 16);
          c = u2f((uint32_t)((const uint16_t*)p.q)[qoff + D / 2 + f] << 16);
        }
        const float x0 = (lb & 1) ? c : a, x1 = (lb & 1) ? -a : c;
        const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
        const _Float16 z = (_Float16)0.f;
        AK[j] = (lb >> 1) ? (half4v){z, z, h0, h1} : (half4v){h0, h1, z, z};
        if constexpr (QF32) {
          const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
          AKl[j] = (lb >> 1) ? (half4v){z, z, l0, l1} : (half4v){l0, l1, z, z};
        }
      }
    }

    // lane constants
    const uint32_t koff = (uint32_t)(lane % NSLOT) * EB;   // K stripe window
    const uint32_t voff = 128u + koff;                       // V stripe window
    const uint32_t asel0 = lb == 0 ? 0x0c0c0100u : (lb == 1 ? 0x01000c0cu : 0x0c0c0c0cu);
    const uint32_t asel1 = lb == 2 ? 0x0c0c0100u : (lb == 3 ? 0x01000c0cu : 0x0c0c0c0cu);
    const int bperm_src = ((lane & 48) | (lb << 2) | la) << 2;  // K-role lane holding my V position
    const int P = 1 << p.log2P;
    const size_t kv_stride = (size_t)P * R;                   // V rows follow the K rows of a page
    const int32_t* btb = p.block_table + (size_t)b * p.max_pages;
    const int NT = p.NT;
    const int gbase = p0 + pgrp * 4;          // first position of this row's group at step 0
    const int lim = min(len, p0 + p.Lc);
    const int last = max(len - 1, 0);
    int steps = lim > gbase ? (lim - gbase + NT - 1) / NT : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) steps = max(steps, __shfl_xor(steps, o));
    steps = __builtin_amdgcn_readfirstlane((steps + 1) & ~1);   // two steps per iteration

    // raw block-table entry of the step's position group (only trusted when len > 0)
    auto page_at = [&](int st) -> int {
      const int gs = min(gbase + st * NT, last);
      return btb[gs >> p.log2P];
    };
    auto row_load = [&](int st, int raw_page, uint32_t* kw, uint32_t* vw) {
      const int page = len > 0 ? raw_page : 0;
      const int g0 = gbase + st * NT;
      const int pk = min(g0 + lb, last), pv = min(g0 + la, last);
      const uint8_t* base = p.cache + ((size_t)page * p.H_kv + h) * 2 * kv_stride;
      RowLoad<LB>::load(base + (size_t)(pk & (P - 1)) * R + la * LB, kw);
      RowLoad<LB>::load(base + kv_stride + (size_t)(pv & (P - 1)) * R + lb * LB, vw);
    };
    // table rows of positions 4g..4g+3 are interleaved: chunk j of quarter la
    // of position 4g + n sits at float4 ((g*FP + j)*4 + la)*4 + n, so the 16
    // lanes of a row (4 positions x 4 quarters) read one contiguous 256-B run
    auto table_load = [&](int st, float4v* tb) {
      const int pk = min(gbase + st * NT + lb, last);
      const float4v* tr = (const float4v*)p.rope + ((size_t)(pk >> 2) * FP * 4 + la) * 4 + (pk & 3);
#pragma unroll
      for (int j = 0; j < FP; ++j) tb[j] = tr[j * 16];
    };

    // gathered K and V slice entries of the current step
    Entry<EB> klo[Q], khi[Q], ve[2 * Q];
    auto gather_k = [&](const uint32_t* kw) {
#pragma unroll
      for (int r = 0; r < Q; ++r) {
        klo[r] = lds_entry<EB>(lds, slot_addr<BITS>(kw, r, koff));
        khi[r] = lds_entry<EB>(lds, slot_addr<BITS>(kw, Q + r, koff));
      }
    };
    auto gather_v = [&](const uint32_t* vw) {
#pragma unroll
      for (int sl = 0; sl < 2 * Q; ++sl) ve[sl] = lds_entry<EB>(lds, slot_addr<BITS>(vw, sl, voff));
    };

    // one decode step.  On entry klo/khi/ve hold the gathers of step st and
    // (kwn, vwn) the index rows of step st+1.  The step gathers step st+1 as
    // soon as the registers free up, then refills (kwn, vwn) with the rows of
    // st+3 (page id pgr, read two steps earlier) and reads the page of st+5.
    // tcur holds the RoPE rows of st; tnext receives those of st+1.
    auto do_step = [&](int st, uint32_t* kwn, uint32_t* vwn, const float4v* tcur, float4v* tnext, int& pgr) {
      const int g0 = gbase + st * NT;
      table_load(st + 1, tnext);

      // ---- K side: X, Y of every frequency pair on the matrix cores (all
      //      issued back to back), then s = sum_f cos_f X_f + sin_f Y_f
      float4v xy[FP];
#pragma unroll
      for (int j = 0; j < FP; ++j) {
        const int r = (2 * j) / C, e = (2 * j) % C;          // entry and element of f = 2j
        const uint32_t w0 = perm(khi[r].d[e >> 1], klo[r].d[e >> 1], 0x05040100u);   // (k_f,  k_h)
        const uint32_t w1 = perm(khi[r].d[e >> 1], klo[r].d[e >> 1], 0x07060302u);   // (k_f', k_h')
        const half4v Bk = __builtin_bit_cast(half4v, (uint2v){w0, w1});
        xy[j] = __builtin_amdgcn_mfma_f32_4x4x4f16(AK[j], Bk, (float4v){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        if constexpr (QF32) xy[j] = __builtin_amdgcn_mfma_f32_4x4x4f16(AKl[j], Bk, xy[j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, QF32 ? 2 * FP : FP, 0);   // the MFMAs first
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int j = 0; j < FP; ++j) {
        const float4v t4 = tcur[j];
        s0 = fmaf(t4.x, xy[j].x, s0);
        s1 = fmaf(t4.y, xy[j].y, s1);
        s0 = fmaf(t4.z, xy[j].z, s0);
        s1 = fmaf(t4.w, xy[j].w, s1);
      }
      float s = s0 + s1;
      // sum over the four quarters (lanes 4 apart within the 16-lane row)
      s += u2f(__builtin_amdgcn_mov_dpp(f2u(s), 0x124, 0xf, 0xf, true));   // row_ror:4
      s += u2f(__builtin_amdgcn_mov_dpp(f2u(s), 0x128, 0xf, 0xf, true));   // row_ror:8
      // to the V role: this lane handles position slot la
      s = u2f(__builtin_amdgcn_ds_bpermute(bperm_src, f2u(s)));
      gather_k(kwn);                                  // K entries of step st+1
      const bool valid = g0 + la < lim;

      // ---- online softmax (log2 domain, lazy max)
      const float s2 = valid ? s * p.scale_log2 : -INFINITY;
      const bool need = s2 > m + LAZY_TAU;
      if (__ballot(need) != 0) {
        if (need) {
          const float fct = __builtin_amdgcn_exp2f(m - s2);
          l *= fct;
          lx *= fct;
#pragma unroll
          for (int u = 0; u < U; ++u) acc[u] *= fct;
          m = s2;
        }
      }
      const float pf = valid ? __builtin_amdgcn_exp2f(s2 - m) : 0.f;
      lx += pf;
      const _Float16 ph = (_Float16)pf;
      const uint32_t pbits = (uint32_t)__builtin_bit_cast(uint16_t, ph);
      const half4v A = __builtin_bit_cast(half4v, (uint2v){perm(0u, pbits, asel0), perm(0u, pbits, asel1)});
      // fp32 output: p = fp16 high part + fp16 low part, two MFMAs per unit
      half4v Alo;
      if constexpr (QF32) {
        const _Float16 pl = (_Float16)(pf - (float)ph);
        const uint32_t lbits = (uint32_t)__builtin_bit_cast(uint16_t, pl);
        Alo = __builtin_bit_cast(half4v, (uint2v){perm(0u, lbits, asel0), perm(0u, lbits, asel1)});
        l += (float)ph + (float)pl;
      } else {
        l += (float)ph;
      }

      // ---- V side: acc += p * v on the matrix cores (block = one token)
#pragma unroll
      for (int sl = 0; sl < 2 * Q; ++sl) {
        if constexpr (EB == 8) {
          const half4v Bv = __builtin_bit_cast(half4v, (uint2v){ve[sl].d[0], ve[sl].d[1]});
          acc[sl] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, Bv, acc[sl], 0, 0, 0);
          if constexpr (QF32) acc[sl] = __builtin_amdgcn_mfma_f32_4x4x4f16(Alo, Bv, acc[sl], 0, 0, 0);
        } else if constexpr (EB == 16) {
          const half4v B0 = __builtin_bit_cast(half4v, (uint2v){ve[sl].d[0], ve[sl].d[1]});
          const half4v B1 = __builtin_bit_cast(half4v, (uint2v){ve[sl].d[2], ve[sl].d[3]});
          acc[2 * sl] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, B0, acc[2 * sl], 0, 0, 0);
          if constexpr (QF32) acc[2 * sl] = __builtin_amdgcn_mfma_f32_4x4x4f16(Alo, B0, acc[2 * sl], 0, 0, 0);
          acc[2 * sl + 1] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, B1, acc[2 * sl + 1], 0, 0, 0);
          if constexpr (QF32) acc[2 * sl + 1] = __builtin_amdgcn_mfma_f32_4x4x4f16(Alo, B1, acc[2 * sl + 1], 0, 0, 0);
        } else if (sl & 1) {
          // two 2-channel entries form one 4-channel unit
          const half4v Bv = __builtin_bit_cast(half4v, (uint2v){ve[sl - 1].d[0], ve[sl].d[0]});
          acc[sl >> 1] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, Bv, acc[sl >> 1], 0, 0, 0);
          if constexpr (QF32) acc[sl >> 1] = __builtin_amdgcn_mfma_f32_4x4x4f16(Alo, Bv, acc[sl >> 1], 0, 0, 0);
        }
      }
      gather_v(vwn);                                  // V entries of step st+1
      row_load(st + 3, pgr, kwn, vwn);
      pgr = page_at(st + 5);
    };

    uint32_t kwA[LW], vwA[LW], kwB[LW], vwB[LW];
    float4v tbA[FP], tbB[FP];
    row_load(0, page_at(0), kwA, vwA);
    row_load(1, page_at(1), kwB, vwB);
    table_load(0, tbA);
    gather_k(kwA);
    gather_v(vwA);
    row_load(2, page_at(2), kwA, vwA);
    int pgB = page_at(3), pgA = page_at(4);
    // an active wave has steps >= 2; the first two steps are peeled so that the
    // loads outstanding at the loop head are in the same order on entry and on
    // the back edge (the wait counts at the head are then tight)
    do_step(0, kwB, vwB, tbA, tbB, pgB);
    do_step(1, kwA, vwA, tbB, tbA, pgA);
    for (int st = 2; st < steps; st += 2) {
      do_step(st, kwB, vwB, tbA, tbB, pgB);
      do_step(st + 1, kwA, vwA, tbB, tbA, pgA);
    }
  }

  // ---- merge the position slots of each (pair, quarter) and write the chunk's partial
  __syncthreads();                       // every wave is done with the slices
  float* red = (float*)lds + (size_t)wave * 64 * SW;
  {
    float* r = red + lane * SW;
#pragma unroll
    for (int u = 0; u < U; ++u) { r[4 * u] = acc[u].x; r[4 * u + 1] = acc[u].y; r[4 * u + 2] = acc[u].z; r[4 * u + 3] = acc[u].w; }
    r[4 * U] = m;
    r[4 * U + 1] = l;
    r[4 * U + 2] = lx;
  }
  __syncthreads();
  // one lane per (pair, quarter): row kslot < NP, position slot la == 0
  if (active && pair_ok && kslot < p.NP && la == 0 && p0 < len) {
    const int nsrc = 4 / p.NP * 4;       // rows of this pair x position slots
    float M = -INFINITY;
    for (int i = 0; i < nsrc; ++i) {
      const int src = (kslot + (i >> 2) * p.NP) * 16 + (i & 3) * 4 + lb;
      const float* r = red + src * SW;
      if (r[4 * U + 1] > 0.f) M = fmaxf(M, r[4 * U]);
    }
    float4v o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) o[u] = (float4v){0.f, 0.f, 0.f, 0.f};
    float L = 0.f, LX = 0.f;
    for (int i = 0; i < nsrc; ++i) {
      const int src = (kslot + (i >> 2) * p.NP) * 16 + (i & 3) * 4 + lb;
      const float* r = red + src * SW;
      if (!(r[4 * U + 1] > 0.f)) continue;
      const float wt = __builtin_amdgcn_exp2f(r[4 * U] - M);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        o[u].x = fmaf(wt, r[4 * u], o[u].x);
        o[u].y = fmaf(wt, r[4 * u + 1], o[u].y);
        o[u].z = fmaf(wt, r[4 * u + 2], o[u].z);
        o[u].w = fmaf(wt, r[4 * u + 3], o[u].w);
      }
      L = fmaf(wt, r[4 * U + 1], L);
      LX = fmaf(wt, r[4 * U + 2], LX);
    }
    const size_t part = (size_t)(h * p.n_pairs + k) * p.n_chunks + ch;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float* op = p.part_o + part * D;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int lc = 4 * u;
      const int base = lc < F ? lb * F + lc : D / 2 + lb * F + (lc - F);
      *(float4v*)(op + base) = o[u] * inv;
    }
    if (lb == 0) p.part_lse[part] = L > 0.f ? M + log2f(LX) : -INFINITY;
  }
}

// ---- combine: one workgroup per (request, query head)
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
  float M = -INFINITY;
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
template <int D, int C, int BITS>
static hipError_t launch_split_t(const DecodeParams& p, bool qf32, int grid, hipStream_t s) {
  if (qf32) hipLaunchKernelGGL((decode_split_kernel<D, C, BITS, true>), dim3(grid), dim3(256), 0, s, p);
  else hipLaunchKernelGGL((decode_split_kernel<D, C, BITS, false>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_decode_split(int D, int C, int bits, bool qf32, const DecodeParams& p, int grid,
                               hipStream_t s) {
#define LVQ_CASE(d, c, b) if (D == d && C == c && bits == b) return launch_split_t<d, c, b>(p, qf32, grid, s);
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
