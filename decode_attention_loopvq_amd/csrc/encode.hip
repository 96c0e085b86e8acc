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
//  * argmin ||z - e||^2 = argmax (z.e - 0.5*||e||^2): the dot products are
//    32x32x16 fp16 MFMAs, one tile of 32 entries x 32 vectors, with
//    -0.5*||e||^2 (read from LDS) as the accumulator input, so the distance
//    needs no VALU work beyond the argmax.
//  * The MFMA reduction index runs over the coupled coordinates in loop-major
//    order (kappa = m*c + i) on both operands, so a lane's operand is c
//    contiguous channels of one loop step (one 8- or 16-byte load).  bf16
//    inputs convert to fp16 exactly inside fp16's normal range; fp32 inputs
//    are split into an fp16 high and low part placed side by side along the
//    reduction index (against two copies of the entry).
//  * A wave scores units of 32 consecutive (token, group) vectors; lane
//    (hf, col) holds vector col and 16 of every tile's 32 entries.  It keeps
//    the tile with the largest maximum (strict compare in increasing tile
//    order) and copies that tile's scores only when the best tile changes;
//    the lowest row at the maximum is found once per unit, and the two lanes
//    of a vector merge with a lexicographic compare (lowest index on ties).
//  * The whole codebook tile set stays in registers for the life of the wave;
//    the raw input loads run three units ahead of the scoring.
//  * The argmax is exact, so it costs VALU work per score (a three-input max
//    per two scores); that VALU work, not the MFMA rate, bounds the kernel.
//  * Near-tie count (NTC, only when the caller asks for it): a vector is a near
//    tie when a second entry scores within 0.5e-6*(||z||^2 + ||e_a||^2) of the
//    best (squared distances within 1e-6 of that scale).  The instance that
//    counts them rescores the vector's tiles after the search and adds the
//    wave's count to one device counter; the plain instance carries none of it.

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace loopvq {

template <int G, int C, bool XF32, int BITS, bool PAGED, bool PG, bool NTC, bool ONE>
__global__ __launch_bounds__(256) void encode_kernel(EncodeParams p) {
  constexpr int KD = XF32 ? 2 * G : G;          // reduction length (fp32: high and low halves)
  constexpr int KDP = KD < 16 ? 16 : KD;        // padded to the MFMA depth
  constexpr int NMF = KDP / 16;                 // 32x32x16 MFMAs per tile
  constexpr int KENT = 1 << BITS;
  constexpr int NTILE = KENT >= 32 ? KENT / 32 : 1;   // 4-bit: one tile, rows 16..31 unused
  constexpr int CH = C < 8 ? C : 8;             // channels per contiguous run of one loop step
  constexpr int NRUN = 8 / CH;                  // runs per lane and MFMA
  constexpr int RW = XF32 ? CH : CH / 2;        // 32-bit words per run

  __shared__ uint16_t cbp[KENT * G];
  // -0.5*||e||^2 of the 16 rows a lane holds per tile, [t][h][16] (h = lane / 32;
  // rows 8q + 4h + s), the MFMA accumulator inputs; -inf on unused rows
  __shared__ __attribute__((aligned(16))) float hsl[NTILE * 2 * 16];

  // work-item and workgroup ids from the hardware registers: this file is
  // built with -mno-amdgpu-ieee, which keeps the device library's id queries
  // from inlining (they would be calls returning per-lane values)
  const int tid = (int)__builtin_amdgcn_workitem_id_x();
  const int bidx = (int)__builtin_amdgcn_workgroup_id_x(), bidy = (int)__builtin_amdgcn_workgroup_id_y();
  const int H = p.H_kv, Tc = p.Tc, D = p.D;
  // y = ((beta*kv_n + kv - kv_lo)*H + hd)*NG + gq: with one codebook per channel group
  // (PG) a workgroup codes group gq only, with that group's codebook
  const int NG = PG ? D / C : 1;
  const int gq = PG ? bidy % NG : 0;
  const int y = PG ? bidy / NG : bidy;
  const int hd = y % H, kv = p.kv_lo + (y / H) % p.kv_n, beta = y / (p.kv_n * H);
  const size_t cbi = ((size_t)(beta * H + hd) * 2 + kv) * NG + gq;   // codebook of this workgroup

  // ---- codebook of (beta, hd, kv), permuted to loop-major coordinates
  const uint16_t* cbsrc = p.cb + cbi * KENT * G;
  for (int x = tid; x < KENT * G; x += 256) {
    const int e = x / G, kap = x - e * G;
    const int m = kap / C, i = kap - m * C;
    cbp[x] = cbsrc[(size_t)e * G + i * Tc + m];
  }
  for (int x = tid; x < NTILE * 32; x += 256) {
    const int t = x >> 5, hh = (x >> 4) & 1, q = (x >> 2) & 3, sr = x & 3;
    const int e = 32 * t + 8 * q + 4 * hh + sr;
    hsl[x] = e < KENT ? -p.hsq[cbi * KENT + e] : -INFINITY;
  }
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hf = lane >> 5, col = lane & 31;

  // ---- entry operands (rows = entries 32t + col, reduction chunk hf), held
  //      for the life of the wave
  half8v A[NTILE][NMF];
#pragma unroll
  for (int t = 0; t < NTILE; ++t)
#pragma unroll
    for (int mu = 0; mu < NMF; ++mu)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kap = 16 * mu + 8 * hf + j;
        const int e = 32 * t + col;
        const uint16_t bits = (kap < KD && e < KENT) ? cbp[e * G + (kap % G)] : (uint16_t)0;
        A[t][mu][j] = __builtin_bit_cast(_Float16, bits);
      }

  const int n = D / C;                 // groups (vectors) per token, a power of two
  const int ln = __builtin_ctz(n);
  const int R = n * BITS / 8;
  const int lr = __builtin_ctz(R);     // row bytes, a power of two
  const int P = 1 << p.log2P;
  const void* xsrc = kv ? p.xv : p.xk;
  const int nvec = PG ? p.n_tok : p.n_tok * n;   // vectors of this stream (PG: of group gq)
  const int nunit = (nvec + 31) >> 5;  // units of 32 vectors
  const int u0 = (bidx * 4 + wave) * p.units_per_wave;
  const int u1 = min(u0 + p.units_per_wave, nunit);
  if (u0 >= u1) return;                // no work (no barrier follows)

  // element offset of run (mu, q) of this lane, without the token/group part
  // element offsets: loop step (beta*Tc + m), head, token.  Dense input is
  // [step][token][head][D]; paged bf16 input is [step][page][head][2][8][D]
  // with token j in page src_slot[j] / 8, slot src_slot[j] % 8
  const size_t step_stride = (size_t)p.step_stride;
  const size_t head_stride = PAGED ? (size_t)16 * D : (size_t)D;
  size_t run_off[NMF][NRUN];
  bool run_ok[NMF][NRUN];
#pragma unroll
  for (int mu = 0; mu < NMF; ++mu)
#pragma unroll
    for (int q = 0; q < NRUN; ++q) {
      const int kap = 16 * mu + 8 * hf + q * CH;
      run_ok[mu][q] = kap < KD;
      const int kp = (XF32 && kap >= G) ? kap - G : kap;
      const int m = kp / C, i0 = kp - m * C;
      run_off[mu][q] = (size_t)(beta * Tc + m) * step_stride + (size_t)hd * head_stride + i0;
    }
  // raw input words of one unit (bf16 pairs or fp32), converted at use
  // (with a unit inside one token, also that token's slot: a scalar load from
  // the constant address space, so its wait never holds on vector loads)
  struct Raw { uint32_t w[NMF][NRUN][RW]; int slot; };
  typedef __attribute__((address_space(4))) const int cint4;
  // dense input with n <= 32 groups per token: a unit is 32/n whole tokens and
  // a lane keeps its group, so its offset advances by a wave-uniform step per
  // unit (no per-lane multiplies); the last, partial unit takes the clamped path
  const bool incr = !PAGED && !PG && ln <= 5;
  const size_t lane_off0 = (size_t)(col >> (ln <= 5 ? ln : 0)) * H * D + (size_t)(col & (n - 1)) * C;
  const size_t unit_step = (size_t)(32 >> (ln <= 5 ? ln : 0)) * H * D;
  auto load_raw = [&](int u, Raw& r) {
    if constexpr (ONE)
      r.slot = ((cint4*)(uintptr_t)p.slot_mapping)[__builtin_amdgcn_readfirstlane((min(u, nunit - 1) << 5) >> ln)];
    size_t voff;
    if (incr && u * 32 + 31 < nvec) {
      voff = lane_off0 + (size_t)u * unit_step;
    } else {
      const int v = min(u * 32 + col, nvec - 1);     // clamped: loads stay in bounds
      const int tok = PG ? v : v >> ln, g = PG ? gq : v & (n - 1);
      size_t tbase;
      if constexpr (PAGED) {
        const int ss = p.src_slot[tok];
        tbase = ((size_t)(ss >> 3) * H * 16 + (ss & 7)) * D;
      } else {
        tbase = (size_t)tok * H * D;
      }
      voff = tbase + (size_t)g * C;
    }
#pragma unroll
    for (int mu = 0; mu < NMF; ++mu)
#pragma unroll
      for (int q = 0; q < NRUN; ++q) {
#pragma unroll
        for (int j = 0; j < RW; ++j) r.w[mu][q][j] = 0u;
        if (!run_ok[mu][q]) continue;
        const size_t off = voff + run_off[mu][q];
        if constexpr (XF32) {
          const float* s = (const float*)xsrc + off;
          if constexpr (CH == 8) {
            const float4v a = *(const float4v*)s, b = *(const float4v*)(s + 4);
            r.w[mu][q][0] = f2u(a.x); r.w[mu][q][1] = f2u(a.y); r.w[mu][q][2] = f2u(a.z); r.w[mu][q][3] = f2u(a.w);
            r.w[mu][q][4] = f2u(b.x); r.w[mu][q][5] = f2u(b.y); r.w[mu][q][6] = f2u(b.z); r.w[mu][q][7] = f2u(b.w);
          } else if constexpr (CH == 4) {
            const float4v a = *(const float4v*)s;
            r.w[mu][q][0] = f2u(a.x); r.w[mu][q][1] = f2u(a.y); r.w[mu][q][2] = f2u(a.z); r.w[mu][q][3] = f2u(a.w);
          } else {
            const uint2v a = *(const uint2v*)s;
            r.w[mu][q][0] = a.x; r.w[mu][q][1] = a.y;
          }
        } else {
          const uint16_t* s = (const uint16_t*)xsrc + off;
          if constexpr (CH == 8) {
            const uint4v a = *(const uint4v*)s;
            r.w[mu][q][0] = a.x; r.w[mu][q][1] = a.y; r.w[mu][q][2] = a.z; r.w[mu][q][3] = a.w;
          } else if constexpr (CH == 4) {
            const uint2v a = *(const uint2v*)s;
            r.w[mu][q][0] = a.x; r.w[mu][q][1] = a.y;
          } else {
            r.w[mu][q][0] = *(const uint32_t*)s;
          }
        }
      }
  };
  // fp16 operand: bf16 values convert exactly; fp32 values are split into a
  // high part (reduction index < G) and a low part (index >= G)
  auto to_operand = [&](const Raw& r, half8v* Bv) {
#pragma unroll
    for (int mu = 0; mu < NMF; ++mu)
#pragma unroll
      for (int q = 0; q < NRUN; ++q)
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const int kap = 16 * mu + 8 * hf + q * CH + j;
          float v;
          if constexpr (XF32) v = u2f(r.w[mu][q][j]);
          else v = (j & 1) ? bf16hi(r.w[mu][q][j >> 1]) : bf16lo(r.w[mu][q][j >> 1]);
          const _Float16 hi = (_Float16)v;
          Bv[mu][q * CH + j] = (XF32 && kap >= G && kap < KD) ? (_Float16)(v - (float)hi) : hi;
        }
  };

  // rows of this (block, head, K|V) stream: page q holds them at q*page_bytes
  // (below 2^32: the boundary rejects larger pages)
  const uint32_t page_bytes = (uint32_t)H * 2u * (uint32_t)(P * R);
  uint8_t* const head_rows = p.cache + (int64_t)beta * p.block_stride + (size_t)(hd * 2 + kv) * P * R;
  // row slot of group g (the row order of the cache; q = n/8 is a power of two)
  const int lq = __builtin_ctz(n >> 3), hgr = n >> 1;
  auto slot_of = [&](int g) {
    const bool hi = g >= hgr;
    const int gg = hi ? g - hgr : g;
    return ((gg >> lq) << (lq + 1)) + (hi ? (1 << lq) : 0) + (gg & ((1 << lq) - 1));
  };
  // a lane's group is fixed when a unit holds whole tokens (n divides 32) or
  // the workgroup codes one group (PG); then so is its row slot
  const bool fixed_group = PG || ln <= 5;
  const int sl_lane = slot_of(PG ? gq : (col & (n - 1)));

  // software pipeline over units: the raw loads of unit u+3 are issued while
  // unit u is scored
  Raw rb[4];
  load_raw(u0, rb[0]);
  load_raw(u0 + 1, rb[1]);
  load_raw(u0 + 2, rb[2]);
  typedef float float16v __attribute__((ext_vector_type(16)));
  auto do_unit = [&](int u, Raw& cur, Raw& nxt) {
    half8v Bv[NMF];
    to_operand(cur, Bv);
    load_raw(u + 3, nxt);
    const int v = u * 32 + col;
    const bool vok = v < nvec;
    const int vc = vok ? v : nvec - 1;
    const int tok = PG ? vc : vc >> ln, g = PG ? gq : vc & (n - 1);
    // with 32 or more groups per token (and one codebook for all groups) a
    // unit lies inside one token, whose slot is then one scalar load and whose
    // row address is scalar arithmetic
    int slot_s = 0, slot_v = 0;
    if constexpr (ONE) slot_s = cur.slot;
    else slot_v = p.slot_mapping[tok];
    // ---- scores against all entries: per 32-entry tile a lane holds 16
    //      entries (rows 8q + 4*hf + s) of its vector.  It keeps the best tile
    //      (strict compare of the tile maxima in increasing tile order) and
    //      that tile's 16 scores; the lowest row holding the maximum is
    //      resolved at the end, so the search takes the lowest index on ties.
    float best = -INFINITY;
    int btile = 0;
    float16v bd;
    // opaque per-unit base: keeps the accumulator-input reads inside the unit
    int hbase = hf * 64;
    __asm__ __volatile__("" : "+v"(hbase));
    // scores of tile t: the MFMA with -0.5*||e||^2 as the accumulator input
    auto tile_scores = [&](int t) {
      const uint8_t* hp = (const uint8_t*)hsl + t * 128 + hbase;
      const float4v c0 = *(const float4v*)hp, c1 = *(const float4v*)(hp + 16);
      const float4v c2 = *(const float4v*)(hp + 32), c3 = *(const float4v*)(hp + 48);
      float16v d = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w,
                    c2.x, c2.y, c2.z, c2.w, c3.x, c3.y, c3.z, c3.w};
#pragma unroll
      for (int mu = 0; mu < NMF; ++mu) d = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[t][mu], Bv[mu], d, 0, 0, 0);
      return d;
    };
    // the running maximum taken over the tile's scores; it grows exactly when
    // the tile's maximum is strictly larger, which makes it the best tile
    auto keep_best = [&](int t, const float16v& d) {
      float m = best;
#pragma unroll
      for (int r = 0; r < 16; r += 2) m = __builtin_fmaxf(__builtin_fmaxf(m, d[r]), d[r + 1]);
      // a masked branch copies the scores (64-bit moves) instead of selecting
      // all 16 every tile; some lane of the wave takes it at almost every tile
      if (m > best) {
        __asm__ __volatile__("");          // keeps this a masked branch (no selects)
        btile = t;
        bd = d;
      }
      best = m;
    };
    // the MFMA of tile t+1 is issued before the search of tile t (whose
    // masked branch ends a basic block), so the matrix core runs during it
    float16v dc = tile_scores(0);
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      float16v dn;
      if (t + 1 < NTILE) dn = tile_scores(t + 1);
      keep_best(t, dc);
      if (t + 1 < NTILE) dc = dn;
    }
    int rr = 15;
#pragma unroll
    for (int r = 14; r >= 0; --r) rr = bd[r] == best ? r : rr;
    int bidx = 32 * btile + 8 * (rr >> 2) + 4 * hf + (rr & 3);
    // ---- merge the two lanes holding the same vector (lower index on ties)
    const float ob = __shfl_xor(best, 32);
    {
      const int oi = __shfl_xor(bidx, 32);
      const bool take = ob > best || (ob == best && oi < bidx);
      bidx = take ? oi : bidx;
    }
    if constexpr (NTC) {
      // near tie: some entry other than the chosen one scores at least
      // best - 0.5e-6*(||z||^2 + ||e_a||^2), i.e. two or more entries do.
      // ||z||^2 from the lane's operand half (fp32 input: the high parts)
      float zz = 0.f;
#pragma unroll
      for (int mu = 0; mu < NMF; ++mu)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int kap = 16 * mu + 8 * hf + j;
          if (kap < G) zz = fmaf((float)Bv[mu][j], (float)Bv[mu][j], zz);
        }
      zz += __shfl_xor(zz, 32);
      // 0.5*||e_a||^2 sits at hsl[t][h][q][s] for entry a = 32t + 8q + 4h + s
      const int hx = ((bidx >> 5) << 5) | (((bidx >> 2) & 1) << 4) | (((bidx >> 3) & 3) << 2) | (bidx & 3);
      const float thr = __builtin_fmaxf(best, ob) - 0.5e-6f * (zz - 2.f * hsl[hx]);
      int cnt = 0;
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        const float16v d = tile_scores(t);
#pragma unroll
        for (int r = 0; r < 16; ++r) cnt += d[r] >= thr ? 1 : 0;
      }
      cnt += __shfl_xor(cnt, 32);
      const uint64_t tied = __ballot(hf == 0 && vok && cnt >= 2);
      if (lane == 0 && tied != 0) atomicAdd(p.near_tie, (int)__popcll(tied));
    }
    // ---- write the code into its row slot
    // byte of the code: page, row in the page (rows are a power of two of
    // bytes), slot byte; unsigned 32-bit parts and one 32 x 32 -> 64 product
    auto row_of = [&](uint32_t us) {
      return head_rows + ((uint64_t)(us >> p.log2P) * page_bytes + ((us & (uint32_t)(P - 1)) << lr));
    };
    auto put = [&](uint8_t* row, uint32_t sl, bool ok) {
      if constexpr (BITS == 8) {
        if (hf == 0 && ok) row[sl] = (uint8_t)bidx;
      } else {
        const int other = __shfl_xor(bidx, 1);
        if (hf == 0 && ok && (col & 1) == 0) row[sl >> 1] = (uint8_t)((bidx & 15) | ((other & 15) << 4));
      }
    };
    if constexpr (ONE) {
      // every vector of the unit exists (the vector count is a multiple of 32)
      put(row_of((uint32_t)slot_s), (uint32_t)(ln == 5 ? sl_lane : slot_of(v & (n - 1))), true);
    } else {
      put(row_of((uint32_t)slot_v), (uint32_t)(fixed_group ? sl_lane : slot_of(g)), vok);
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

template <int G, int C, bool XF32, int BITS, bool PG>
static hipError_t launch_encode_pg(const EncodeParams& p, int n_blocks, hipStream_t s) {
  dim3 grid(p.n_unit_groups, n_blocks * p.kv_n * p.H_kv * (PG ? p.D / C : 1));
  // 32 or more groups per token (one codebook for all): a unit of 32 vectors
  // lies inside one token
  const bool one = !PG && p.D / C >= 32;
  if constexpr (!XF32) {
    // bf16 window pages (decode-time page encoding); no near-tie count there
    if (p.src_slot != nullptr) {
      if (p.near_tie != nullptr) return hipErrorInvalidValue;
      if (one) hipLaunchKernelGGL((encode_kernel<G, C, XF32, BITS, true, PG, false, !PG>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((encode_kernel<G, C, XF32, BITS, true, PG, false, false>), grid, dim3(256), 0, s, p);
      return hipGetLastError();
    }
  }
  if (p.src_slot != nullptr) return hipErrorInvalidValue;
  if (p.near_tie != nullptr)
    hipLaunchKernelGGL((encode_kernel<G, C, XF32, BITS, false, PG, true, false>), grid, dim3(256), 0, s, p);
  else if (one)
    hipLaunchKernelGGL((encode_kernel<G, C, XF32, BITS, false, PG, false, !PG>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((encode_kernel<G, C, XF32, BITS, false, PG, false, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int G, int C, bool XF32, int BITS>
static hipError_t launch_encode_t(const EncodeParams& p, int n_blocks, hipStream_t s) {
  if constexpr (BITS == 8) {
    if (p.per_group) return launch_encode_pg<G, C, XF32, BITS, true>(p, n_blocks, s);
  }
  if (p.per_group) return hipErrorInvalidValue;
  return launch_encode_pg<G, C, XF32, BITS, false>(p, n_blocks, s);
}

hipError_t launch_encode(int G, bool xf32, int bits, const EncodeParams& p, int n_blocks, hipStream_t s) {
  const int c = p.c;
#define LVQ_ENC(g, cc, f, b) \
  if (G == g && c == cc && xf32 == f && bits == b) return launch_encode_t<g, cc, f, b>(p, n_blocks, s);
#define LVQ_ENC_C(g, f, b) LVQ_ENC(g, 2, f, b) LVQ_ENC(g, 4, f, b) LVQ_ENC(g, 8, f, b)
  LVQ_ENC_C(16, false, 8) LVQ_ENC_C(32, false, 8) LVQ_ENC_C(16, false, 4) LVQ_ENC_C(32, false, 4)
  LVQ_ENC_C(8, true, 8) LVQ_ENC_C(16, true, 8) LVQ_ENC_C(32, true, 8)
  LVQ_ENC_C(8, true, 4) LVQ_ENC_C(16, true, 4) LVQ_ENC_C(32, true, 4)
  // G channels of one loop step (c = G, Tc = 1): the baseline grouping
  LVQ_ENC(16, 16, false, 8) LVQ_ENC(16, 16, true, 8)
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
