// Quantised split-K decode attention for LoopVQ on gfx950.
//
// What it computes [LoopVQ paper, hub.valency.io/works/W_7srt5hed_v1,
// section "System implementation", attention; appendix
// "Optimizing pre-RoPE vector quantization serving efficiency"]: at loop step t every
// cached token j of a request contributes its key rebuilt from the step's
// codebook slice, rotated by RoPE at position j, and its value rebuilt the
// same way; tokens are cut into splits, and joining the splits' partial
// softmax outputs by log-sum-exp (the combine kernel) yields exactly the
// softmax over all tokens.
//
// MI355X mapping (this file's own design, not the pages'):
//  * A workgroup is eight waves on one KV head.  The head's K and V slices are
//    staged once in LDS, every entry replicated over a 256-byte row (one copy
//    per bank window), and lane l reads window l mod (256 / entry bytes):
//    random code gathers of a wave then hit each of the 64 banks once per
//    pass.  A gather address is one v_perm_b32 (code -> byte 1, lane window
//    -> byte 0, K|V region -> byte 2).
//  * A wave serves a duo of (request, query head) pairs 2i and 2i+1 over a
//    chunk of positions, 16 positions per step.  When the GQA group is even
//    the duo's pairs are query heads of one request and share one index
//    stream and its key gathers.  With a GQA group that is a multiple of
//    four (G4) a wave serves a quad, pairs 4i .. 4i+3, all query heads of one
//    request and KV head: one index stream, one set of key gathers, and each
//    V lane accumulates two query heads from one set of value gathers.  As
//    the four heads share each key, the lane rotates the key once (fp32, 4
//    VALU operations per frequency instead of 8 for four heads) and the dot
//    products with the four queries run as fp32 v_mfma_f32_4x4x1f32 products
//    (row = head, column = position), issued after the rotations into two
//    accumulators that are summed once.
//  * K side: a lane owns one position (of its 16-lane row) and one quarter
//    of the RoPE frequencies.  For each frequency one v_mfma_f32_4x4x4f16 with
//    the block-diagonal query matrix [[q0_f, q0_h], [q0_h, -q0_f]] (+) the same
//    for pair 1 and the key column (k0_f, k0_h, k1_f, k1_h) yields
//    X = q_f k_f + q_h k_h and Y = q_h k_f - q_f k_h of both pairs with exact
//    fp16 products; the lane then adds cos*X + sin*Y in fp32, which equals
//    q . RoPE(k).  One load of cos/sin serves both pairs.
//  * V side: rows 0-1 of the wave serve pair 0, rows 2-3 pair 1; a lane takes
//    two positions and one channel quarter, and the same MFMA with A = p*I
//    and the gathered V entries as B accumulates p*v in fp32 registers.
//  * Online softmax in the log2 domain with a lazy maximum: the running max
//    is only raised when a score exceeds it by more than 8 (so p <= 256).
//  * RoPE rows come from a table interleaved by groups of 4 positions (one
//    contiguous 256-byte run per 16 lanes); with eight duos per head the
//    workgroup stages each step's rows once into an LDS ring (see below).
//  * TaSQ-coded keys (TQ) [appendix "Orthogonal application with TaSQ",
//    "Formulation" and "Grouping under loop coupling"]: the codes index
//    u = P(w k / sigma), whose codes hold whole RoPE pairs (u channels 2p,
//    2p+1 = key channels perm[p], perm[p] + D/2).  The lane's frequencies
//    become the u pairs of its quarter's groups: one 32-bit word of an entry is
//    the (f, f + D/2) pair of a key column, so no byte perms are needed.  The
//    channel weights fold into the query operand, which is then no longer an
//    fp16 value: the MFMA's reduction index carries it as an fp16 high and low
//    part against the same pair twice, A row = (x_f hi, x_h hi, x_f lo, x_h lo)
//    and B column = (u_f, u_h, u_f, u_h), so products stay exact and one MFMA
//    covers both pairs of a duo when they share keys.  P reorders the RoPE
//    frequencies: the shared rows are written into the LDS ring in the head's
//    frequency order (two 8-byte stores per staged piece, at offsets fixed for
//    the kernel's life), and per-wave rows are read by 8-byte loads at fixed
//    per-lane offsets.  sigma multiplies each score in the V role; it is
//    loaded with the step's V index rows.
#pragma once

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
    // byte 1 <- code; bytes 0 and 2 <- lane offset (window, K|V region); byte 3 <- 0
    return perm(w[s >> 2], lane_off, 0x0c020000u | ((4u + (s & 3)) << 8));
  } else {
    uint32_t code = (w[s >> 3] >> ((s & 7) * 4)) & 15u;
    return (code << 8) | lane_off;
  }
}

// one codebook per channel group: LDS address of the entry whose code sits in
// slot s of the lane's row words.  The lane's quarter is folded into base; slot
// s < Q is group base_group + s, slot Q + r its RoPE partner N/2 + base_group + r,
// and entry e of group g sits at (g*KENT + e)*EB (no replication)
template <int BITS, int EB, int KENT, int Q, int N>
__device__ __forceinline__ uint32_t slot_addr_pg(const uint32_t* w, int s, uint32_t base) {
  uint32_t code;
  if constexpr (BITS == 8) code = (w[s >> 2] >> ((s & 3) * 8)) & 255u;
  else code = (w[s >> 3] >> ((s & 7) * 4)) & 15u;
  const int gc = s < Q ? s : N / 2 + s - Q;
  return code * EB + base + (uint32_t)(gc * KENT * EB);
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

template <int D, int C, int BITS, bool QF32, bool SHARE, bool SP, bool ST, bool PG, bool TQ, bool G4>
__global__ __launch_bounds__(512, 1) void decode_split_kernel(DecodeParams p) {
  static_assert(!G4 || (SHARE && SP && !QF32 && !PG && !TQ), "quads: one request per wave, bf16 queries, pages of 16+");
  constexpr int N = D / C;            // groups per row
  constexpr int Q = N / 8;            // lo (and hi) groups per lane quarter
  constexpr int F = D / 8;            // RoPE frequencies per lane quarter (one K MFMA each)
  constexpr int FP = F / 2;           // float4 table words per quarter (two frequencies each)
  constexpr int EB = 2 * C;           // bytes of one slice entry
  constexpr int NWIN = 256 / EB;      // bank windows per 256-byte LDS row (64 banks)
  constexpr int R = N * BITS / 8;     // row bytes
  constexpr int LB = R / 4;           // row bytes per lane quarter
  constexpr int LW = (LB + 3) / 4;    // row words per lane
  constexpr int U = D / 16;           // 4-channel V units per lane and pair
  constexpr int KENT = 1 << BITS;
  constexpr int NS = SHARE ? 1 : 2;   // index streams per wave: the duo's requests
  constexpr int NT = 16;              // positions per wave step
  constexpr int PW = G4 ? 4 : 2;      // (request, query head) pairs per wave
  constexpr int HPL = G4 ? 2 : 1;     // query heads per V lane
  constexpr int WAVES = 8;            // waves per workgroup, all on one KV head
  constexpr int TSTEP = NT * D * 4;   // bytes of the RoPE rows of one step
  // slices: shared codebook, every entry replicated over a 256-byte row;
  // one codebook per group (PG), the N*KENT entries of each of K and V packed
  constexpr int LDS_SLICES = PG ? 2 * N * KENT * EB : 2 * KENT * 256;
  constexpr int LDS_RING = ST ? 2 * TSTEP : 0;
  constexpr int PGMAX = DECODE_PAGE_LIST;   // page-list entries per stream and wave (shared rows)
  constexpr int LDS_PAGES = ST ? WAVES * 2 * PGMAX * 4 : 0;
  constexpr int LDS_BYTES = LDS_SLICES + LDS_RING + LDS_PAGES;
  // quads put the ring and the page lists first, so that their per-step
  // reads carry the whole offset in the instruction (below 64 KiB) and the
  // slice gathers take the slices' base the same way (measured: 1% faster
  // for quads, 2% slower for duos, which keep the slices first)
  constexpr int OFF_SL = G4 ? LDS_RING + LDS_PAGES : 0;
  constexpr int OFF_RING = G4 ? 0 : LDS_SLICES;
  constexpr int OFF_PAGES = OFF_RING + LDS_RING;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  uint8_t* const lds_sl = lds + OFF_SL;
  __shared__ int wsteps[WAVES];
  __shared__ int tqinv[TQ ? D / 2 : 1];     // TaSQ: u pair of each RoPE frequency
  // G4: requests in order of decreasing coded length (ties by index), so that
  // the eight quads of a workgroup, which it runs in step, have similar lengths
  __shared__ int req_sorted[G4 ? DECODE_SORT_MAX : 1];
  __shared__ __attribute__((aligned(16))) int len_sorted[G4 ? DECODE_SORT_MAX : 1];
  __shared__ int wg_busy;
  __shared__ int wg_item[2];                // G4 with shared rows: (group of 8 quads, chunk)

  // ---- workgroup -> (KV head, 8 work items).  Heads vary fastest, so each
  //      XCD (blocks of one residue mod 8, renumbered contiguously) owns a
  //      band of chunks of every head: its L2 holds only that band's RoPE rows.
  //      Quads (ragged GQA batches, whose chunks and requests differ in work)
  //      keep the hardware's interleaving instead: every XCD then gets an
  //      equal share of long and short work items, and the workgroups, which
  //      come in order of decreasing work, are handed out as CUs free up.
  int bid = blockIdx.x;
  const int nb = gridDim.x;
  if (!G4 && (nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int wgi = bid / p.H_kv;
  const int h = bid - wgi * p.H_kv;

  // ---- G4: rank the requests by length (every workgroup computes the same
  //      order from seq_lens), then leave at once if none of this workgroup's
  //      quads has positions in its chunk (nothing staged, nothing written)
  const bool sorted = G4 && p.B <= DECODE_SORT_MAX;
  // with shared rows (eight quads per workgroup, one chunk) the workgroups
  // take the (group of 8 quads, chunk) items in order of decreasing work: a
  // group is 8 quads in length order, its work in chunk c is
  // clamp(L - c*Lc, 0, Lc) positions (L its longest request).  Full chunks
  // come first (group-major), then each group's last, partial chunk by
  // decreasing size.  A workgroup keeps its head's slices in LDS and takes
  // the items of ranks item_rank(0), item_rank(1), ... of its head: w,
  // 2S - 1 - w, 2S + w, ... for workgroup w of the S of its head, which
  // deals the items out largest first and evens out the workgroups' sums
  const bool ordered = G4 && ST && sorted && p.n_dg / WAVES <= 64;
  const int wg_stride = max(nb / p.H_kv, 1);   // workgroups per head (quads keep the hardware's order)
  auto item_rank = [&](int r) { return r * wg_stride + ((r & 1) ? wg_stride - 1 - wgi : wgi); };
  // wave 0 writes the (group, chunk) of the item of rank `it` to wg_item
  // (group -1: no such item)
  auto select_item = [&](int it) {
    if constexpr (!G4) return;
    if (threadIdx.x < 64) {
      const int n_groups = p.n_dg / WAVES;
      const int g = (int)threadIdx.x;
      const int qpr = p.grp >> 2;
      const int Lg = g < n_groups ? len_sorted[req_sorted[(WAVES * g) / qpr]] : 0;
      const int fc = Lg / p.Lc, pr = Lg - fc * p.Lc;
      // inclusive prefix of the full-chunk counts over the groups
      int inc = fc;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(inc, d);
        if (g >= d) inc += o;
      }
      const int FT = __shfl(inc, 63);
      bool mine;
      int cg;
      if (it < FT) {
        mine = it >= inc - fc && it < inc;
        cg = it - (inc - fc);
      } else {
        // partial chunks: rank by (size desc, group asc)
        int rank = 0;
#pragma unroll
        for (int o = 0; o < 64; ++o) {
          const int po = __builtin_amdgcn_readlane(pr, o);
          rank += (po > pr || (po == pr && o < g)) ? 1 : 0;
        }
        mine = pr > 0 && rank == it - FT;
        cg = fc;
      }
      const uint64_t bal = __ballot(mine);
      const int src = bal ? (int)__builtin_ctzll(bal) : 0;
      const int cs = __shfl(cg, src);
      if (g == 0) {
        wg_item[0] = bal ? src : -1;
        wg_item[1] = bal ? cs : 0;
      }
    }
  };
  if constexpr (G4) {
    if (sorted) {
      // lengths padded with -1 to a multiple of 4 (padding ranks after every request)
      const int B4 = (p.B + 3) & ~3;
      for (int t = threadIdx.x; t < B4; t += WAVES * 64)
        len_sorted[t] = t < p.B ? min(max(p.seq_lens[t], 0), p.max_seq_len) : -1;
      __syncthreads();
      for (int t = threadIdx.x; t < p.B; t += WAVES * 64) {
        const int lt = len_sorted[t];
        int r = 0;
        for (int j = 0; j < B4; j += 4) {
          const int4 lj = *(const int4*)(len_sorted + j);
          r += (lj.x > lt || (lj.x == lt && j < t)) ? 1 : 0;
          r += (lj.y > lt || (lj.y == lt && j + 1 < t)) ? 1 : 0;
          r += (lj.z > lt || (lj.z == lt && j + 2 < t)) ? 1 : 0;
          r += (lj.w > lt || (lj.w == lt && j + 3 < t)) ? 1 : 0;
        }
        req_sorted[r] = t;
      }
    }
    if (threadIdx.x == 0) wg_busy = 0;
    __syncthreads();
    if (ordered) {
      select_item(item_rank(0));
      __syncthreads();
      if (wg_item[0] < 0) return;   // workgroup-uniform: no work left for this item number
    } else {
      if (threadIdx.x < WAVES) {
        const int it = wgi * WAVES + (int)threadIdx.x;
        if (it < p.items_per_head) {
          const int c0 = it / p.n_dg, qd = it - c0 * p.n_dg;
          const int bs = qd / (p.grp >> 2);
          const int b = sorted ? req_sorted[bs] : bs;
          if (c0 * p.Lc < min(max(p.seq_lens[b], 0), p.max_seq_len)) atomicOr(&wg_busy, 1);
        }
      }
      __syncthreads();
      if (wg_busy == 0) return;   // workgroup-uniform
    }
  }

  // ---- stage the K and V slices of head h, each entry replicated over a
  //      256-byte row (one copy per bank window): entry e of region kv sits
  //      at kv*KENT*256 + e*256, and lane l reads window l % NWIN, so the
  //      random gathers of a wave hit every bank once per pass
  // Each thread's loads are all issued before its LDS stores (fixed trip
  // counts, unrolled): a load-store loop waits one L2 round trip per pass.
  constexpr int NTHR = WAVES * 64;
  if constexpr (PG) {
    // one codebook per channel group: the head's [2][N][KENT] entries as they
    // are (random gathers then meet bank conflicts; 256-byte replication of
    // N*KENT entries would not fit in LDS)
    constexpr int NV = LDS_SLICES / 16, BATCH = 8;
    static_assert(NV % (NTHR * BATCH) == 0, "slice copy: whole batches per thread");
    const uint4v* src = (const uint4v*)((const uint8_t*)p.slices + (size_t)h * LDS_SLICES);
    for (int x0 = 0; x0 < NV; x0 += NTHR * BATCH) {
      uint4v v[BATCH];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) v[j] = src[x0 + j * NTHR + threadIdx.x];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) ((uint4v*)lds_sl)[x0 + j * NTHR + threadIdx.x] = v[j];
    }
  } else {
    // 16 threads per entry, one 16-byte piece of its 256-byte row each
    constexpr int NIT = 2 * KENT * 16 / NTHR;
    static_assert(2 * KENT * 16 == NIT * NTHR, "slice copy: whole passes per thread");
    const uint8_t* src = (const uint8_t*)p.slices + (size_t)h * 2 * KENT * EB;
    uint4v v[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int ke = (it * NTHR + (int)threadIdx.x) >> 4;   // ke = kv * KENT + e
      const uint8_t* sp = src + (size_t)ke * EB;
      if constexpr (EB == 16) {
        v[it] = *(const uint4v*)sp;
      } else if constexpr (EB == 8) {
        uint2v t = *(const uint2v*)sp; v[it] = (uint4v){t.x, t.y, t.x, t.y};
      } else {
        uint32_t t = *(const uint32_t*)sp; v[it] = (uint4v){t, t, t, t};
      }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int x = it * NTHR + (int)threadIdx.x;
      *(uint4v*)(lds_sl + (x >> 4) * 256 + (x & 15) * 16) = v[it];
    }
  }
  if constexpr (TQ) {
    // inverse of the head's pair permutation (out-of-range entries are ignored)
    if (threadIdx.x < D / 2) {
      const int f = p.tq_perm[h * (D / 2) + threadIdx.x];
      if ((unsigned)f < (unsigned)(D / 2)) tqinv[f] = threadIdx.x;
    }
  }
  __syncthreads();

  // ---- the workgroup's items: one, or with ordered items every item of
  //      ranks item_rank(0), item_rank(1), ... (the slices stay in LDS)
  for (int rnd = 0;; ++rnd) {
    // ---- this wave's work item (wave-uniform): one duo of pairs, one chunk
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    // G4 with shared rows and ordered items: group wg_item[0], chunk wg_item[1]
    const int item = ordered ? (wg_item[1] * p.n_dg + wg_item[0] * WAVES + wave) : wgi * WAVES + wave;
    const bool item_ok = item < p.items_per_head;
    const int ch = item_ok ? item / p.n_dg : 0;
    const int duo = item_ok ? item - ch * p.n_dg : 0;
    const int row = lane >> 4;                 // position group of this 16-lane row
    const int la = (lane >> 2) & 3, lb = lane & 3;
    // K role: quarter la, position slot lb.  V role: position slot la, quarter lb.
    // coded positions of stream s: [lo[s], len[s]) (positions below lo[s] are
    // a bf16 sink attended elsewhere); has[s]: the stream has coded positions
    int kq[2], bq[2], len[2], lo[2];
    bool okq[2], has[2];
    // G4: the quad's first pair (its request taken in length order)
    int pair0 = PW * duo;
    if constexpr (G4) {
      const int qpr = p.grp >> 2;                  // quads per request
      const int bs = duo / qpr;
      pair0 = (sorted ? req_sorted[min(bs, p.B - 1)] : bs) * p.grp + (duo - bs * qpr) * 4;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      kq[s] = pair0 + s;
      okq[s] = item_ok && kq[s] < p.n_pairs;
      bq[s] = okq[s] ? kq[s] / p.grp : 0;
      len[s] = okq[s] ? min(max(p.seq_lens[bq[s]], 0), p.max_seq_len) : 0;
      lo[s] = (okq[s] && p.seq_lo != nullptr) ? min(max(p.seq_lo[bq[s]], 0), len[s]) : 0;
      has[s] = lo[s] < len[s];
    }
    // G4: pairs 2 and 3 of the quad (the same request as pairs 0 and 1)
    bool okq_hi[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) okq_hi[s] = G4 && item_ok && pair0 + 2 + s < p.n_pairs;
    const int p0 = ch * p.Lc;
    const int lenx = max(len[0], len[1]);
    const bool active = item_ok && p0 < lenx;   // wave-uniform

    // V role: rows 0-1 of the wave serve pair 0 and rows 2-3 pair 1 (G4: pairs
    // 0, 1 and pairs 2, 3); a lane takes the adjacent positions 8*rp + 2*la and
    // 8*rp + 2*la + 1 of the step and channel quarter lb
    const int sv = row >> 1, rp = row & 1;
    float m[HPL], l[HPL], lx[HPL];         // running max (log2 domain); sum of the rounded p
                                           // used in the products; exact sum of p (logsumexp)
    float4v acc[HPL][U];
#pragma unroll
    for (int j = 0; j < HPL; ++j) {
      m[j] = -INFINITY;
      l[j] = 0.f;
      lx[j] = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) acc[j][u] = (float4v){0.f, 0.f, 0.f, 0.f};
    }

    // ---- K-side A operands (read by active waves only).  For frequency f (the
    //      i-th of quarter la) lane lb supplies row lb of the block-diagonal
    //        [[q0_f, q0_h, 0, 0], [q0_h, -q0_f, 0, 0], [0, 0, q1_f, q1_h], [0, 0, q1_h, -q1_f]]
    //      (q_h = q_{f + D/2}; pair 0 and pair 1 of the duo), so that with the
    //      key column (k0_f, k0_h, k1_f, k1_h) of a position the MFMA yields
    //      X0, Y0, X1, Y1 of that position.
    //      fp32 queries (QF32): the same row of each pair, each coefficient as an
    //      fp16 high and low part along the reduction index, A row =
    //      (x_f hi, x_h hi, x_f lo, x_h lo) against the key column
    //      (k_f, k_h, k_f, k_h) of one stream, so one product covers both pairs
    //      when they share keys and two (one per stream) when they do not.
    half4v AK[G4 ? 1 : F];
    //      G4: the quad's four query heads share one key per position, so the
    //      lane rotates that key itself (fp32) and the matrix cores take the
    //      dot products with fp32 operands: lane lb supplies head lb's query
    //      at the quarter's channels f (AQ[i]) and f + D/2 (AQ[F + i]), one
    //      v_mfma_f32_4x4x1f32 per channel against the rotated key's channel
    float AQ[G4 ? 2 * F : 1];
    // TaSQ: u pair of the lane's i-th frequency slot: the pairs of its quarter's
    // lo groups, then those of its hi groups
    auto tq_upair = [&](int i) { return i < F / 2 ? la * (F / 2) + i : D / 4 + la * (F / 2) + (i - F / 2); };
    auto tq_freq = [&](int i) { return min(max(p.tq_perm[h * (D / 2) + tq_upair(i)], 0), D / 2 - 1); };
    if (active && TQ) {
      // row lb of the block-diagonal query matrix over (u_f, u_h) with the
      // weights folded in, [[q0_f/w_f, q0_h/w_h], [q0_h/w_f, -q0_f/w_h]] (+) pair 1,
      // each coefficient as fp16 high and low parts along the reduction index
      const int s = lb >> 1;
      const int kk = s ? kq[1] : kq[0], bb = s ? bq[1] : bq[0];
      const int jq = h * p.grp + (okq[s] ? kk - bb * p.grp : 0);
      const size_t qrow = ((size_t)bb * p.H_q + jq) * D;
      const float* wrow = p.tq_w + (size_t)h * D;
#pragma unroll
      for (int i = 0; i < F; ++i) {
        const int f = tq_freq(i);
        float a, c;
        if constexpr (QF32) {
          a = ((const float*)p.q)[qrow + f];
          c = ((const float*)p.q)[qrow + f + D / 2];
        } else {
          a = u2f((uint32_t)((const uint16_t*)p.q)[qrow + f] << 16);
          c = u2f((uint32_t)((const uint16_t*)p.q)[qrow + f + D / 2] << 16);
        }
        const float x0 = ((lb & 1) ? c : a) / wrow[f];
        const float x1 = ((lb & 1) ? -a : c) / wrow[f + D / 2];
        const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
        AK[i] = (half4v){h0, h1, (_Float16)(x0 - (float)h0), (_Float16)(x1 - (float)h1)};
      }
    } else if (active) {
      const int s = lb >> 1;
      const int kk = s ? kq[1] : kq[0], bb = s ? bq[1] : bq[0];
      const int jq = h * p.grp + (okq[s] ? kk - bb * p.grp : 0);
      const size_t qoff = ((size_t)bb * p.H_q + jq) * D + la * F;
      if constexpr (G4) {
        // head lb of the quad: pair kq[lb & 1] + (lb & 2), clamped to a valid
        // head of the request when past the group's end
        const bool okh = (lb & 2) ? ((lb & 1) ? okq_hi[1] : okq_hi[0]) : ((lb & 1) ? okq[1] : okq[0]);
        const int kh = ((lb & 1) ? kq[1] : kq[0]) + (lb & 2), bh = (lb & 1) ? bq[1] : bq[0];
        const int jh = h * p.grp + (okh ? kh - bh * p.grp : 0);
        const size_t qh = ((size_t)bh * p.H_q + jh) * D + la * F;
#pragma unroll
        for (int i = 0; i < F; ++i) {
          AQ[i] = u2f((uint32_t)((const uint16_t*)p.q)[qh + i] << 16);
          AQ[F + i] = u2f((uint32_t)((const uint16_t*)p.q)[qh + D / 2 + i] << 16);
        }
      } else {
#pragma unroll
        for (int i = 0; i < F; ++i) {
          float a, c;
          if constexpr (QF32) {
            a = ((const float*)p.q)[qoff + i];
            c = ((const float*)p.q)[qoff + D / 2 + i];
          } else {
            a = u2f((uint32_t)((const uint16_t*)p.q)[qoff + i] << 16);
            c = u2f((uint32_t)((const uint16_t*)p.q)[qoff + D / 2 + i] << 16);
          }
          const float x0 = (lb & 1) ? c : a, x1 = (lb & 1) ? -a : c;
          const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
          const _Float16 z = (_Float16)0.f;
          if constexpr (QF32) {
            AK[i] = (half4v){h0, h1, (_Float16)(x0 - (float)h0), (_Float16)(x1 - (float)h1)};
          } else {
            AK[i] = s ? (half4v){z, z, h0, h1} : (half4v){h0, h1, z, z};
          }
        }
      }
    }

    // ---- lane constants
    // K window / V window in LDS (PG: the lane quarter's first group of K / V)
    const uint32_t koff = PG ? (uint32_t)(la * Q * KENT * EB) : (uint32_t)(lane % NWIN) * EB;
    const uint32_t voff = PG ? (uint32_t)((N + lb * Q) * KENT * EB) : (uint32_t)(KENT * 256) + koff;
    const uint32_t asel0 = lb == 0 ? 0x0c0c0100u : (lb == 1 ? 0x01000c0cu : 0x0c0c0c0cu);
    const uint32_t asel1 = lb == 2 ? 0x0c0c0100u : (lb == 3 ? 0x01000c0cu : 0x0c0c0c0cu);
    // the same for the high half of a packed pair of fp16 values
    const uint32_t asel2 = lb == 0 ? 0x0c0c0302u : (lb == 1 ? 0x03020c0cu : 0x0c0c0c0cu);
    const uint32_t asel3 = lb == 2 ? 0x0c0c0302u : (lb == 3 ? 0x03020c0cu : 0x0c0c0c0cu);
    // K-role lanes holding my V positions 8*rp + 2*la (+1): row 2*rp + la/2,
    // position slots 2*(la%2) (+1); quarters 2*sv, 2*sv + 1 expose pair sv's
    // score after the quarter sum
    const int bperm_a = ((16 * (2 * rp + (la >> 1))) | ((2 * sv + (lb & 1)) << 2) | (2 * (la & 1))) << 2;
    const int bperm_b = bperm_a + 4;
    // G4: K-role lane of quarter la exposes pair la; my heads 2*sv + j at my
    // two positions sit at quarter 2*sv + j, slots 2*(la%2) (+1)
    const int bperm_g4 = ((16 * (2 * rp + (la >> 1))) | ((2 * sv) << 2) | (2 * (la & 1))) << 2;
    const int P = 1 << p.log2P;
    const uint32_t kv_stride = (uint32_t)(P * R);             // V rows follow the K rows of a page
    // bytes between pages (below 2^32: the boundary rejects larger strides), so
    // a page's offset is one 32 x 32 -> 64-bit product of unsigned values
    const uint32_t page_stride = (uint32_t)p.H_kv * 2u * kv_stride;
    const uint8_t* head_base = p.cache + (size_t)h * 2 * kv_stride;
    // pages of 8 positions: wave-uniform page ids (two per stream and step, see
    // page_at) except with TaSQ keys, whose per-wave-row path keeps per-lane page
    // ids (uniform ones cost it more registers than it has)
    constexpr bool P8U = !SP && !TQ;
    // byte offsets of the lane's K and V row quarters from the first row of the
    // step (the whole step inside one page, SP), of the lane's page (P8U:
    // positions 0-7 of a step in one page, 8-15 in the next), or of the lane's
    // own 4-position row group
    const uint32_t kro = (uint32_t)(((SP ? 4 * row : (P8U ? 4 * (row & 1) : 0)) + lb) * R + la * LB);
    const uint32_t vro = kv_stride + (uint32_t)(((SP ? 8 * rp : 0) + 2 * la) * R + lb * LB);   // +R: slot b
    const uint32_t tbo = (uint32_t)((row * FP * 16 + la * 4 + lb) * 16);
    int lim[2], last[2];
    const int32_t* btb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      lim[s] = min(len[s], p0 + p.Lc);
      last[s] = max(len[s] - 1, 0);
      btb[s] = p.block_table + (size_t)bq[s] * p.max_pages;
    }
    const int limx = max(lim[0], lim[1]);
    // the V lane's positions 8*rp + 2*la (+1) of a step, relative to lo, and the
    // span [lo, lim) of coded positions in this chunk
    const int vrel = 8 * rp + 2 * la - lo[sv];
    const uint32_t vspan = (uint32_t)max(lim[sv] - lo[sv], 0);
    const int glast = (max(last[0], last[1]) >> 4) << 4;   // last step-aligned group with data
    const int my_steps = active ? (limx - p0 + NT - 1) / NT : 0;   // wave-uniform
    // an opaque zero: keeps the page-id loads on the vector path, in order
    // with the row loads (scalar loads would share a counter with the LDS gathers)
    const int vz = (int)__builtin_amdgcn_mbcnt_lo(0u, 0u);

    // raw block-table entries of the step's pages (only trusted when the
    // stream's length is positive).  SP: one per stream, wave-uniform.  P8U: two
    // per stream, wave-uniform, the page of the step's positions 0-7 and that
    // of 8-15 (a step starts on a multiple of 16).  Else per lane, one per
    // stream for the K row group and one for the V groups
    constexpr int NPG = SP ? NS : (P8U ? 2 * NS : NS + 1);
    auto page_at = [&](int st, int* pg) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if constexpr (SP) {
          pg[s] = btb[s][(min(max(p0 + st * NT, lo[s]), last[s]) >> p.log2P) + vz];
        } else if constexpr (P8U) {
          pg[2 * s] = btb[s][(min(max(p0 + st * NT, lo[s]), last[s]) >> p.log2P) + vz];
          pg[2 * s + 1] = btb[s][(min(max(p0 + st * NT + 8, lo[s]), last[s]) >> p.log2P) + vz];
        } else {
          pg[s] = btb[s][min(max(p0 + st * NT + 4 * row, lo[s]), last[s]) >> p.log2P];
        }
      }
      if constexpr (!SP && !P8U) pg[NS] = btb[sv][min(max(p0 + st * NT + 8 * rp, lo[sv]), last[sv]) >> p.log2P];
    };
    // K rows of both streams at the lane's K position, V rows of stream sv at
    // the lane's two V positions
    // (TaSQ: also the fp16 sigma of the lane's two V positions, issued before
    // the V rows so that waiting for the rows covers them)
    auto row_load = [&](int st, const int* raw_page, uint32_t (*kw)[LW], uint32_t (*vw)[LW], uint32_t& sg) {
      const uint8_t* vbase;
      size_t vslot;                               // first slot of the V rows' group (page*P + offset)
      if constexpr (SP) {
        const uint8_t* base[2];
        size_t slot0[2];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const uint32_t page = has[s] ? (uint32_t)__builtin_amdgcn_readfirstlane(raw_page[s]) : 0u;
          const uint32_t gs = (uint32_t)(min(p0 + st * NT, last[s]) & ~(NT - 1)) & (uint32_t)(P - 1);
          base[s] = head_base + ((uint64_t)page * page_stride + gs * (uint32_t)R);
          slot0[s] = (size_t)page * P + gs + 8 * rp;
          RowLoad<LB>::load(base[s] + kro, kw[s]);
        }
        vbase = (NS == 1 || sv == 0) ? base[0] : base[NS - 1];
        vslot = (NS == 1 || sv == 0) ? slot0[0] : slot0[NS - 1];
      } else if constexpr (P8U) {
        // page A holds the step's positions 0-7 (K rows of lane rows 0-1, V rows
        // of rp = 0), page B positions 8-15; both start at row 0 of their page.
        // Past the end of a stream both clamp to its last page (rows read there
        // are in bounds and masked)
        const uint8_t* vb[2];
        size_t vs[2];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const uint32_t pga = has[s] ? (uint32_t)__builtin_amdgcn_readfirstlane(raw_page[2 * s]) : 0u;
          const uint32_t pgb = has[s] ? (uint32_t)__builtin_amdgcn_readfirstlane(raw_page[2 * s + 1]) : 0u;
          const uint8_t* ba = head_base + (uint64_t)pga * page_stride;
          const uint8_t* bb = head_base + (uint64_t)pgb * page_stride;
          RowLoad<LB>::load((row >= 2 ? bb : ba) + kro, kw[s]);
          vb[s] = rp ? bb : ba;
          vs[s] = (size_t)(rp ? pgb : pga) * P;
        }
        vbase = (NS == 1 || sv == 0) ? vb[0] : vb[NS - 1];
        vslot = (NS == 1 || sv == 0) ? vs[0] : vs[NS - 1];
      } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const uint32_t page = has[s] ? (uint32_t)raw_page[s] : 0u;
          const uint32_t gs = (uint32_t)(min(p0 + st * NT + 4 * row, last[s]) & ~3) & (uint32_t)(P - 1);
          RowLoad<LB>::load(head_base + ((uint64_t)page * page_stride + gs * (uint32_t)R) + kro, kw[s]);
        }
        const uint32_t page = has[sv] ? (uint32_t)raw_page[NS] : 0u;
        const uint32_t gs = (uint32_t)(min(p0 + st * NT + 8 * rp, last[sv]) & ~7) & (uint32_t)(P - 1);
        vbase = head_base + ((uint64_t)page * page_stride + gs * (uint32_t)R);
        vslot = (size_t)page * P + gs;
      }
      if constexpr (TQ) {
        // the two positions are adjacent: one 4-byte load (the slot is even)
        sg = *(const uint32_t*)(p.tq_sigma + vslot + 2 * la);
      }
      RowLoad<LB>::load(vbase + vro, vw[0]);
      RowLoad<LB>::load(vbase + vro + R, vw[1]);
    };
    // table rows of positions 4g..4g+3 are interleaved: chunk j of quarter la
    // of position 4g + n sits at float4 ((g*FP + j)*4 + la)*4 + n, so the 16
    // lanes of a row (4 positions x 4 quarters) read one contiguous 256-B run,
    // and the rows of one step form one contiguous TSTEP-byte block
    float4v tb[FP];
    // TaSQ, per-wave rows: byte offsets of the lane's frequency slots 2j, 2j+1
    // inside its row of the interleaved table (low / high 16 bits)
    uint32_t toff[(TQ && !ST) ? FP : 1];
    if constexpr (TQ && !ST) {
      auto off = [&](int i) {
        const int f = tq_freq(i);
        return (uint32_t)(((f % F) >> 1) * 256 + (f / F) * 64 + (f & 1) * 8);
      };
#pragma unroll
      for (int j = 0; j < FP; ++j) toff[j] = off(2 * j) | (off(2 * j + 1) << 16);
    }
    const uint32_t tbo_row = (uint32_t)((row * FP * 16 + lb) * 16);
    auto table_load = [&](int st) {
      const int gt = min(p0 + st * NT, glast);
      if constexpr (TQ && !ST) {
        const uint8_t* tr = (const uint8_t*)p.rope + (size_t)(gt >> 2) * FP * 256 + tbo_row;
#pragma unroll
        for (int j = 0; j < FP; ++j) {
          const float2v a = *(const float2v*)(tr + (toff[j] & 0xffffu));
          const float2v b = *(const float2v*)(tr + (toff[j] >> 16));
          tb[j] = (float4v){a.x, a.y, b.x, b.y};
        }
      } else {
        const float4v* tr = (const float4v*)((const uint8_t*)p.rope + (size_t)(gt >> 2) * FP * 256 + tbo);
#pragma unroll
        for (int j = 0; j < FP; ++j) tb[j] = tr[j * 16];
      }
    };

    auto entry_addr = [&](const uint32_t* w, int s, uint32_t off) {
      if constexpr (PG) return slot_addr_pg<BITS, EB, KENT, Q, N>(w, s, off);
      else return slot_addr<BITS>(w, s, off);
    };
    // gathered K slice entries per stream, V entries per V position slot
    Entry<EB> klo[NS][Q], khi[NS][Q], ve[2][2 * Q];
    auto gather_k = [&](uint32_t (*kw)[LW]) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < Q; ++r) {
          klo[s][r] = lds_entry<EB>(lds_sl, entry_addr(kw[s], r, koff));
          khi[s][r] = lds_entry<EB>(lds_sl, entry_addr(kw[s], Q + r, koff));
        }
    };
    auto gather_v = [&](uint32_t (*vw)[LW]) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int sl = 0; sl < 2 * Q; ++sl) ve[t][sl] = lds_entry<EB>(lds_sl, entry_addr(vw[t], sl, voff));
    };

    // ---- K side of a step: X, Y of both pairs for every frequency on the
    //      matrix cores, then s = sum_f cos_f X_f + sin_f Y_f in fp32 (this
    //      lane's quarter; klo/khi and tb hold the step's entries and rows)
    auto k_side = [&](float* sc) {
      const float4v zero = {0.f, 0.f, 0.f, 0.f};
      if constexpr (G4) {
        // rotate the position's key (lo channel f, hi channel f + D/2 of each
        // frequency) in fp32, then add AQ . RoPE(k) for the four heads on the
        // matrix cores: row = head, column = position, one channel per
        // product.  All rotations come first and the products follow, the
        // lo-channel and hi-channel products in two accumulators (one wait
        // state between the paired MFMAs, 4 adds to sum them): an MFMA that
        // waits for the rotation just before it stalls the wave, and one
        // accumulator makes a chain of dependent MFMAs.
        float rf[F], rh[F];
#pragma unroll
        for (int i = 0; i < F; ++i) {
          const int r = i / C, e = i % C;                      // entry and element of frequency i
          const half2v wl = as_h2(klo[0][r].d[e >> 1]), wh = as_h2(khi[0][r].d[e >> 1]);
          const float kf = (float)((e & 1) ? wl.y : wl.x), kh = (float)((e & 1) ? wh.y : wh.x);
          const float cs = (i & 1) ? tb[i >> 1].z : tb[i >> 1].x;
          const float sn = (i & 1) ? tb[i >> 1].w : tb[i >> 1].y;
          rf[i] = fmaf(cs, kf, fmaf(-sn, kh, 0.f));          // RoPE(k)_f
          rh[i] = fmaf(sn, kf, fmaf(cs, kh, 0.f));           // RoPE(k)_{f + D/2}
        }
        float4v a0 = zero, a1 = zero;
#pragma unroll
        for (int i = 0; i < F; ++i) {
          a0 = __builtin_amdgcn_mfma_f32_4x4x1f32(AQ[i], rf[i], a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_4x4x1f32(AQ[F + i], rh[i], a1, 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x002, 4 * F, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * F, 0);
#pragma unroll
        for (int k = 0; k < 4; ++k) sc[k] = a0[k] + a1[k];
      } else {
        float sa0 = 0.f, sb0 = 0.f, sa1 = 0.f, sb1 = 0.f;
#pragma unroll
        for (int i = 0; i < F; ++i) {
          float4v xy;
          if constexpr (TQ) {
            // u pair i of the quarter: word e of entry r of the lo (first F/2) or
            // hi groups holds (u_f, u_h)
            constexpr int PE = C / 2;
            const bool hq = i >= F / 2;
            const int r = (hq ? i - F / 2 : i) / PE, e = (hq ? i - F / 2 : i) % PE;
            const uint32_t w0 = hq ? khi[0][r].d[e] : klo[0][r].d[e];
            xy = __builtin_amdgcn_mfma_f32_4x4x4f16(AK[i], __builtin_bit_cast(half4v, (uint2v){w0, w0}), zero, 0, 0, 0);
            if constexpr (!SHARE) {
              // pair 1 reads its own keys: rows 2-3 of a second product
              const uint32_t w1 = hq ? khi[NS - 1][r].d[e] : klo[NS - 1][r].d[e];
              const float4v xy1 =
                  __builtin_amdgcn_mfma_f32_4x4x4f16(AK[i], __builtin_bit_cast(half4v, (uint2v){w1, w1}), zero, 0, 0, 0);
              xy.z = xy1.z;
              xy.w = xy1.w;
            }
          } else {
            const int r = i / C, e = i % C;                      // entry and element of frequency i
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t w0 = perm(khi[0][r].d[e >> 1], klo[0][r].d[e >> 1], sel);   // (k0_f, k0_h)
            const uint32_t w1 = SHARE ? w0 : perm(khi[NS - 1][r].d[e >> 1], klo[NS - 1][r].d[e >> 1], sel);
            if constexpr (QF32) {
              // rows 0-1 (pair 0) against stream 0's key, rows 2-3 against stream 1's
              xy = __builtin_amdgcn_mfma_f32_4x4x4f16(AK[i], __builtin_bit_cast(half4v, (uint2v){w0, w0}), zero, 0, 0, 0);
              if constexpr (!SHARE) {
                const float4v xy1 =
                    __builtin_amdgcn_mfma_f32_4x4x4f16(AK[i], __builtin_bit_cast(half4v, (uint2v){w1, w1}), zero, 0, 0, 0);
                xy.z = xy1.z;
                xy.w = xy1.w;
              }
            } else {
              xy = __builtin_amdgcn_mfma_f32_4x4x4f16(AK[i], __builtin_bit_cast(half4v, (uint2v){w0, w1}), zero, 0, 0, 0);
            }
          }
          const float cs = (i & 1) ? tb[i >> 1].z : tb[i >> 1].x;
          const float sn = (i & 1) ? tb[i >> 1].w : tb[i >> 1].y;
          sa0 = fmaf(cs, xy.x, sa0);
          sb0 = fmaf(sn, xy.y, sb0);
          sa1 = fmaf(cs, xy.z, sa1);
          sb1 = fmaf(sn, xy.w, sb1);
        }
        // interleave: each MFMA is followed by VALU work (the next perms and this
        // frequency's FMAs); issuing all MFMAs first would hold every X, Y live
        constexpr int KMF = (TQ || QF32) ? (SHARE ? 1 : 2) : 1;
        constexpr int KVALU = TQ ? 4 : 6;
#pragma unroll
        for (int i = 0; i < F; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, KMF, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, KVALU, 0);
        }
        sc[0] = sa0 + sb0;
        sc[1] = sa1 + sb1;
      }
    };
    // sum over the four quarters (lanes 4 apart within the 16-lane row); lanes
    // of quarters 0-1 then expose pair 0's score and quarters 2-3 pair 1's, and
    // each V lane pulls its two positions of its pair
    auto to_v_role = [&](const float* sc, float* sv2) {
      if constexpr (G4) {
        // quarter la exposes pair la; the V lane pulls pairs 2*sv, 2*sv + 1 at
        // its two positions: sv2[2*j + e] = score of head j at position e
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[k] = sc[k];
          v[k] += u2f(__builtin_amdgcn_mov_dpp(f2u(v[k]), 0x124, 0xf, 0xf, true));   // row_ror:4
          v[k] += u2f(__builtin_amdgcn_mov_dpp(f2u(v[k]), 0x128, 0xf, 0xf, true));   // row_ror:8
        }
        const uint32_t ex = f2u(la == 0 ? v[0] : (la == 1 ? v[1] : (la == 2 ? v[2] : v[3])));
#pragma unroll
        for (int k = 0; k < 4; ++k) sv2[k] = u2f(__builtin_amdgcn_ds_bpermute(bperm_g4 + 16 * (k >> 1) + 4 * (k & 1), ex));
        return;
      }
      float v0 = sc[0], v1 = sc[1];
      v0 += u2f(__builtin_amdgcn_mov_dpp(f2u(v0), 0x124, 0xf, 0xf, true));   // row_ror:4
      v1 += u2f(__builtin_amdgcn_mov_dpp(f2u(v1), 0x124, 0xf, 0xf, true));
      v0 += u2f(__builtin_amdgcn_mov_dpp(f2u(v0), 0x128, 0xf, 0xf, true));   // row_ror:8
      v1 += u2f(__builtin_amdgcn_mov_dpp(f2u(v1), 0x128, 0xf, 0xf, true));
      const uint32_t ex = f2u(la >= 2 ? v1 : v0);
      sv2[0] = u2f(__builtin_amdgcn_ds_bpermute(bperm_a, ex));
      sv2[1] = u2f(__builtin_amdgcn_ds_bpermute(bperm_b, ex));
    };
    // ---- online softmax of pair sv at the lane's two positions (log2 domain,
    //      lazy max) and the V side: acc += p * v on the matrix cores (block =
    //      one token); p is rounded to fp16 for the product, and l adds the same
    //      rounded p, so the output stays an exact convex combination
    auto v_side = [&](int g0, const float* sv2, uint32_t sg) {
      const int posa = g0 + vrel;
      const bool va = (uint32_t)posa < vspan, vb = (uint32_t)(posa + 1) < vspan;
#pragma unroll
      for (int j = 0; j < HPL; ++j) {      // G4: the lane's two query heads share the V gathers
        float s0 = sv2[2 * j], s1 = sv2[2 * j + 1];
        if constexpr (TQ) {
          // the rebuilt key is sigma * P^-1(u_hat) / w: the score scales by sigma
          s0 *= (float)as_h2(sg).x;
          s1 *= (float)as_h2(sg).y;
        }
        const float sa = va ? s0 * p.scale_log2 : -INFINITY;
        const float sb = vb ? s1 * p.scale_log2 : -INFINITY;
        const float smax = fmaxf(sa, sb);
        const bool need = smax > m[j] + LAZY_TAU;
        if (__ballot(need) != 0) {
          if (need) {
            // a state with no position yet (m = -inf) holds zeros: only m moves
            if (m[j] != -INFINITY) {
              const float fct = __builtin_amdgcn_exp2f(m[j] - smax);
              l[j] *= fct;
              lx[j] *= fct;
#pragma unroll
              for (int u = 0; u < U; ++u) acc[j][u] *= fct;
            }
            m[j] = smax;
          }
        }
        const float pa = va ? __builtin_amdgcn_exp2f(sa - m[j]) : 0.f;
        const float pb = vb ? __builtin_amdgcn_exp2f(sb - m[j]) : 0.f;
        lx[j] += pa + pb;
        half4v A[2], Alo[2];
        if constexpr (QF32) {
          const float pv[2] = {pa, pb};
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const _Float16 ph = (_Float16)pv[t];
            const uint32_t pbits = (uint32_t)__builtin_bit_cast(uint16_t, ph);
            A[t] = __builtin_bit_cast(half4v, (uint2v){perm(0u, pbits, asel0), perm(0u, pbits, asel1)});
            // fp32 output: p = fp16 high part + fp16 low part, two MFMAs per unit
            const _Float16 pl = (_Float16)(pv[t] - (float)ph);
            const uint32_t lbits = (uint32_t)__builtin_bit_cast(uint16_t, pl);
            Alo[t] = __builtin_bit_cast(half4v, (uint2v){perm(0u, lbits, asel0), perm(0u, lbits, asel1)});
            l[j] += (float)ph + (float)pl;
          }
        } else {
          // both p rounded to fp16 in one packed word; l adds the same two
          // values with one dot product against (1, 1)
          const half2v ph2 = (half2v){(_Float16)pa, (_Float16)pb};
          const uint32_t pw = __builtin_bit_cast(uint32_t, ph2);
          A[0] = __builtin_bit_cast(half4v, (uint2v){perm(0u, pw, asel0), perm(0u, pw, asel1)});
          A[1] = __builtin_bit_cast(half4v, (uint2v){perm(0u, pw, asel2), perm(0u, pw, asel3)});
          l[j] = __builtin_amdgcn_fdot2(ph2, (half2v){(_Float16)1.f, (_Float16)1.f}, l[j], false);
        }
        float4v* ac = acc[j];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int sl = 0; sl < 2 * Q; ++sl) {
            if constexpr (EB == 8) {
              const half4v Bv = __builtin_bit_cast(half4v, (uint2v){ve[t][sl].d[0], ve[t][sl].d[1]});
              ac[sl] = __builtin_amdgcn_mfma_f32_4x4x4f16(A[t], Bv, ac[sl], 0, 0, 0);
              if constexpr (QF32) ac[sl] = __builtin_amdgcn_mfma_f32_4x4x4f16(Alo[t], Bv, ac[sl], 0, 0, 0);
            } else if constexpr (EB == 16) {
              const half4v B0 = __builtin_bit_cast(half4v, (uint2v){ve[t][sl].d[0], ve[t][sl].d[1]});
              const half4v B1 = __builtin_bit_cast(half4v, (uint2v){ve[t][sl].d[2], ve[t][sl].d[3]});
              ac[2 * sl] = __builtin_amdgcn_mfma_f32_4x4x4f16(A[t], B0, ac[2 * sl], 0, 0, 0);
              if constexpr (QF32) ac[2 * sl] = __builtin_amdgcn_mfma_f32_4x4x4f16(Alo[t], B0, ac[2 * sl], 0, 0, 0);
              ac[2 * sl + 1] = __builtin_amdgcn_mfma_f32_4x4x4f16(A[t], B1, ac[2 * sl + 1], 0, 0, 0);
              if constexpr (QF32) ac[2 * sl + 1] = __builtin_amdgcn_mfma_f32_4x4x4f16(Alo[t], B1, ac[2 * sl + 1], 0, 0, 0);
            } else if (sl & 1) {
              // two 2-channel entries form one 4-channel unit
              const half4v Bv = __builtin_bit_cast(half4v, (uint2v){ve[t][sl - 1].d[0], ve[t][sl].d[0]});
              ac[sl >> 1] = __builtin_amdgcn_mfma_f32_4x4x4f16(A[t], Bv, ac[sl >> 1], 0, 0, 0);
              if constexpr (QF32) ac[sl >> 1] = __builtin_amdgcn_mfma_f32_4x4x4f16(Alo[t], Bv, ac[sl >> 1], 0, 0, 0);
            }
          }
        }
      }
    };

    if constexpr (!ST) {
      // ================= per-wave RoPE rows (any batch shape)
      if (active) {
        const int steps = (my_steps + 1) & ~1;   // two steps per iteration
        // one decode step.  On entry klo/khi/ve hold the gathers of step st, tb
        // the RoPE rows of st, and (kwn, vwn) the index rows of step st+1.  The
        // step reloads tb for st+1 and gathers step st+1 as soon as the
        // registers free up, then refills (kwn, vwn) with the rows of st+3
        // (page ids pgr, read two steps earlier) and reads the pages of st+5.
        // (TaSQ: sigma of a step travels with its index rows, and moves to sgc
        // when the step's V entries are gathered, before the rows are refilled)
        uint32_t sgc = 0u;
        auto do_step = [&](int st, uint32_t (*kwn)[LW], uint32_t (*vwn)[LW], uint32_t& sgn, int* pgr) {
          float sc[PW], sv2[2 * HPL];
          k_side(sc);
          table_load(st + 1);                             // RoPE rows of step st+1
          to_v_role(sc, sv2);
          gather_k(kwn);                                  // K entries of step st+1
          v_side(p0 + st * NT, sv2, sgc);
          gather_v(vwn);                                  // V entries of step st+1
          if constexpr (TQ) sgc = sgn;
          row_load(st + 3, pgr, kwn, vwn, sgn);
          page_at(st + 5, pgr);
        };
        uint32_t kwA[NS][LW], vwA[2][LW], kwB[NS][LW], vwB[2][LW];
        uint32_t sgA = 0u, sgB = 0u;
        int pgA[NPG], pgB[NPG], pg0[NPG];
        page_at(0, pg0);
        row_load(0, pg0, kwA, vwA, sgA);
        page_at(1, pg0);
        row_load(1, pg0, kwB, vwB, sgB);
        table_load(0);
        gather_k(kwA);
        gather_v(vwA);
        if constexpr (TQ) sgc = sgA;
        page_at(2, pg0);
        row_load(2, pg0, kwA, vwA, sgA);
        page_at(3, pgB);
        page_at(4, pgA);
        // an active wave has steps >= 2; the first two steps are peeled so that
        // the loads outstanding at the loop head are in the same order on entry
        // and on the back edge (the wait counts at the head are then tight)
        do_step(0, kwB, vwB, sgB, pgB);
        do_step(1, kwA, vwA, sgA, pgA);
        for (int st = 2; st < steps; st += 2) {
          do_step(st, kwB, vwB, sgB, pgB);
          do_step(st + 1, kwA, vwA, sgA, pgA);
        }
      }
    } else {
      // ================= RoPE rows shared by the workgroup.  The eight waves
      // work on one chunk (eight duos of one head), so each step's TSTEP bytes
      // of rows are fetched once per workgroup, one 16-byte piece per lane of
      // each wave, into a two-slot LDS ring, and read back by every wave.  The
      // workgroup moves in lockstep (one barrier per step); waves whose duo has
      // fewer steps keep staging rows for the others.
      // the chunk's block-table entries of each stream, copied once into LDS
      // (read back per step with no long-lived registers): entry i of stream s
      // is the page of index pa[s] + i
      int* plist = (int*)(lds + OFF_PAGES) + wave * 2 * PGMAX;
      // the page of position x is list entry clamp(x, lo, last) / P - pa,
      // capped at pcnt - 1; clamping commutes with the shift, so per step it is
      // min(max(x / P - pa, plo), phi) with one shift shared by the streams
      int pa[2], plo[2], phi[2];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        pa[s] = min(max(p0, lo[s]), last[s]) >> p.log2P;
        const int pcnt = max(min((min(p0 + p.Lc - 1, last[s]) >> p.log2P) - pa[s] + 1, PGMAX), 1);
        plo[s] = (lo[s] >> p.log2P) - pa[s];
        phi[s] = min((last[s] >> p.log2P) - pa[s], pcnt - 1);
        for (int i = lane; i < pcnt; i += 64) plist[s * PGMAX + i] = has[s] ? btb[s][pa[s] + i] : 0;
      }
      if (lane == 0) wsteps[wave] = my_steps;
      __syncthreads();
      int nst = 0;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) nst = max(nst, wsteps[w]);
      nst = (nst + 3) & ~3;                    // four steps per iteration (ring x row buffers)
      constexpr int PIECES = TSTEP / 16 / WAVES;   // 16-byte pieces per wave and step
      const int glast_st = (max(p.max_seq_len - 1, 0) >> 4) << 4;
      float4v sb[2];                           // staged pieces in flight
      auto stage_load = [&](int st, float4v& dst) {
        const int gt = min(p0 + st * NT, glast_st);
        if (lane < PIECES) dst = ((const float4v*)p.rope)[(size_t)(gt >> 2) * FP * 16 + wave * PIECES + lane];
      };
      // TaSQ: the piece's two frequencies go to the slots of their u pairs, so
      // that the ring holds the rows in this head's frequency order
      uint32_t sd0 = 0, sd1 = 0;
      if constexpr (TQ) {
        const int pc = wave * PIECES + lane;
        const int n_ = pc & 3, la_ = (pc >> 2) & 3, j_ = (pc >> 4) % FP, row_ = (pc >> 4) / FP;
        auto dest = [&](int f) {
          const int pp = min(max(tqinv[f], 0), D / 2 - 1);   // in range even for a bad permutation
          const bool hq = pp >= D / 4;
          const int pr = hq ? pp - D / 4 : pp;
          const int la2 = pr / (F / 2), i2 = (hq ? F / 2 : 0) + pr % (F / 2);
          return (uint32_t)((((row_ * FP + (i2 >> 1)) * 4 + la2) * 4 + n_) * 16 + (i2 & 1) * 8);
        };
        sd0 = dest(la_ * F + 2 * j_);
        sd1 = dest(la_ * F + 2 * j_ + 1);
      }
      auto stage_store = [&](int st, const float4v& v) {
        if (lane < PIECES) {
          uint8_t* ring = lds + OFF_RING + (st & 1) * TSTEP;
          if constexpr (TQ) {
            *(float2v*)(ring + sd0) = (float2v){v.x, v.y};
            *(float2v*)(ring + sd1) = (float2v){v.z, v.w};
          } else {
            *(float4v*)(ring + (wave * PIECES + lane) * 16) = v;
          }
        }
      };
      auto table_lds = [&](int st) {
        const uint8_t* ring = lds + OFF_RING + (st & 1) * TSTEP + tbo;
#pragma unroll
        for (int j = 0; j < FP; ++j) tb[j] = *(const float4v*)(ring + j * 256);
      };
      // this wave's LDS writes are done, then the workgroup meets
      auto wg_barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0), other counters untouched
        __asm__ __volatile__("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ __volatile__("" ::: "memory");
      };
      // page ids of step st (uniform values, clamped into the chunk's list)
      auto page_lds = [&](int st, int* pg) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
          pg[s] = plist[s * PGMAX + min(max(((p0 + st * NT) >> p.log2P) - pa[s], plo[s]), phi[s])];
      };
      uint32_t kw[4][NS][LW], vw[4][2][LW], sg[4] = {0u, 0u, 0u, 0u};
      int pgn[NS];                             // page ids of step st+3, read during step st-1
      // one step: index rows of step x live in row buffer x % 4, staged pieces
      // alternate with b2 = st % 2.  Every global load of a step (staged rows,
      // index rows of st+3) and the page-id read are issued on every path and
      // before the step's own work, so the number of operations younger than
      // any awaited one is the same whether or not the wave still has steps:
      // the wait counts stay loose (a wave waits for loads issued steps ago,
      // never for the ones it has just issued).  Scheduling fences keep the
      // phases in order, which bounds the live registers.
      auto st_step = [&](int st, int b4, int b2) {
        wg_barrier();                                   // ring slot st&1 holds the rows of st
        stage_load(st + 2, sb[b2]);
        row_load(st + 3, pgn, kw[(b4 + 3) & 3], vw[(b4 + 3) & 3], sg[(b4 + 3) & 3]);
        page_lds(st + 4, pgn);
        __builtin_amdgcn_sched_barrier(0);
        if (st < my_steps) {
          float sc[PW], sv2[2 * HPL];
          table_lds(st);
          k_side(sc);
          __builtin_amdgcn_sched_barrier(0);
          gather_v(vw[b4]);                             // V entries of step st
          __builtin_amdgcn_sched_barrier(0);
          to_v_role(sc, sv2);
          gather_k(kw[(b4 + 1) & 3]);                   // K entries of step st+1
          __builtin_amdgcn_sched_barrier(0);
          v_side(p0 + st * NT, sv2, sg[b4]);
          __builtin_amdgcn_sched_barrier(0);
        }
        stage_store(st + 1, sb[1 - b2]);
      };
      if (nst > 0) {
        stage_load(0, sb[0]);
        stage_load(1, sb[1]);
        {
          int pg[NS];
          page_lds(0, pg);
          row_load(0, pg, kw[0], vw[0], sg[0]);
          page_lds(1, pg);
          row_load(1, pg, kw[1], vw[1], sg[1]);
          page_lds(2, pg);
          row_load(2, pg, kw[2], vw[2], sg[2]);
          page_lds(3, pgn);
        }
        if (my_steps > 0) gather_k(kw[0]);
        stage_store(0, sb[0]);
        for (int st = 0; st < nst; st += 4) {
          st_step(st, 0, 0);
          st_step(st + 1, 1, 1);
          st_step(st + 2, 2, 0);
          st_step(st + 3, 3, 1);
        }
      }
    }

    // ---- merge the 8 position slots of each (pair, quarter) and write the
    //      chunk's partials.  The slots of one (pair, quarter) are the lanes of
    //      rows 2*sv, 2*sv + 1 at slots la = 0..3 of one quarter lb: 4 and 8
    //      lanes apart inside a row and 16 apart across the two rows.  The
    //      merged state has M = the largest m of the 8 slots and sums weighted
    //      by 2^(m - M) (0 for an empty slot: l = 0, m = -inf).  Three exchange
    //      rounds (DPP row rotations by 4 and 8, then a swizzle that swaps the
    //      two rows) give M in each lane; each lane scales its own state once,
    //      and three more rounds add the scaled states, the rotations fused
    //      into the adds.  Every wave merges its own lanes: no barrier, no LDS.
    auto xchg = [&](float v, int round) -> float {
      if (round == 0) return u2f(__builtin_amdgcn_mov_dpp(f2u(v), 0x124, 0xf, 0xf, true));   // row_ror:4
      if (round == 1) return u2f(__builtin_amdgcn_mov_dpp(f2u(v), 0x128, 0xf, 0xf, true));   // row_ror:8
      return u2f(__builtin_amdgcn_ds_swizzle(f2u(v), 0x401f));                                // lane ^ 16
    };
    float mm[HPL];
#pragma unroll
    for (int j = 0; j < HPL; ++j) {
      float M = m[j];
#pragma unroll
      for (int round = 0; round < 3; ++round) M = fmaxf(M, xchg(M, round));
      const float w = l[j] > 0.f ? __builtin_amdgcn_exp2f(m[j] - M) : 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) acc[j][u] *= w;
      l[j] *= w;
      lx[j] *= w;
      mm[j] = M;
    }
#pragma unroll
    for (int round = 0; round < 3; ++round) {
#pragma unroll
      for (int j = 0; j < HPL; ++j) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float4v a = acc[j][u];
          a.x += xchg(a.x, round);
          a.y += xchg(a.y, round);
          a.z += xchg(a.z, round);
          a.w += xchg(a.w, round);
          acc[j][u] = a;
        }
        l[j] += xchg(l[j], round);
        lx[j] += xchg(lx[j], round);
      }
    }
#pragma unroll
    for (int j = 0; j < HPL; ++j) m[j] = l[j] > 0.f ? mm[j] : -INFINITY;
    // one lane per (pair, quarter) writes: row 2*sv, position slot la == 0
    // (G4: for each of its two query heads, pairs 2*sv and 2*sv + 1 of the quad)
#pragma unroll
    for (int j = 0; j < HPL; ++j) {
      const int pj = G4 ? 2 * sv + j : sv;                   // pair of the wave
      const bool ok0 = (pj & 1) ? okq[1] : okq[0], ok1 = (pj & 1) ? okq_hi[1] : okq_hi[0];
      const bool okj = G4 ? ((pj & 2) ? ok1 : ok0) : (sv ? okq[1] : okq[0]);
      if (!(active && okj && rp == 0 && la == 0 && p0 < (G4 || sv == 0 ? len[0] : len[1]))) continue;
      const int kpair = G4 ? pair0 + pj : kq[sv];
      const size_t part = (size_t)(h * p.n_pairs + kpair) * p.n_chunks + ch;
      const float L = l[j];
      const float inv = L > 0.f ? 1.f / L : 0.f;
      float* op = p.part_o + part * D;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int lc = 4 * u;
        const int base = lc < F ? lb * F + lc : D / 2 + lb * F + (lc - F);
        *(float4v*)(op + base) = acc[j][u] * inv;
      }
      if (lb == 0) p.part_lse[part] = L > 0.f ? m[j] + log2f(lx[j]) : -INFINITY;
    }
    if (!ordered) break;
    // every wave is done with the ring, the page lists and wg_item
    __syncthreads();
    select_item(item_rank(rnd + 1));
    __syncthreads();
    if (wg_item[0] < 0) break;   // workgroup-uniform
  }
}

// ---------------------------------------------------------------- launchers
template <int D, int C, int BITS, bool QF32, bool SHARE, bool PG, bool TQ>
static void launch_split_sp(const DecodeParams& p, int grid, hipStream_t s) {
  // a step's 16 positions lie in one page when pages hold at least 16
  // positions; workgroup-shared RoPE rows need eight duos per head
  if (p.log2P < 4) {
    hipLaunchKernelGGL((decode_split_kernel<D, C, BITS, QF32, SHARE, false, false, PG, TQ, false>), dim3(grid),
                       dim3(512), 0, s, p);
    return;
  }
  if constexpr (!QF32) {
    if (p.shared_rope) {
      hipLaunchKernelGGL((decode_split_kernel<D, C, BITS, false, SHARE, true, true, PG, TQ, false>), dim3(grid),
                         dim3(512), 0, s, p);
      return;
    }
  }
  hipLaunchKernelGGL((decode_split_kernel<D, C, BITS, QF32, SHARE, true, false, PG, TQ, false>), dim3(grid),
                     dim3(512), 0, s, p);
}

template <int D, int C, int BITS, bool PG, bool TQ>
static hipError_t launch_split_t(const DecodeParams& p, bool qf32, int grid, hipStream_t s) {
  // pairs 2i and 2i+1 belong to one request when the GQA group size is even
  const bool share = (p.grp & 1) == 0;
  if constexpr (!PG && !TQ) {
    // quads: four query heads of one request per wave (the split plan sets
    // this for bf16 queries, pages of 16 or more and a group of 4, 8, ...)
    if (p.quad) {
      if (qf32 || p.log2P < 4 || (p.grp & 3) != 0) return hipErrorInvalidValue;
      if (p.shared_rope)
        hipLaunchKernelGGL((decode_split_kernel<D, C, BITS, false, true, true, true, false, false, true>), dim3(grid),
                           dim3(512), 0, s, p);
      else
        hipLaunchKernelGGL((decode_split_kernel<D, C, BITS, false, true, true, false, false, false, true>), dim3(grid),
                           dim3(512), 0, s, p);
      return hipGetLastError();
    }
  }
  if (p.quad) return hipErrorInvalidValue;
  if (qf32) {
    if (share) launch_split_sp<D, C, BITS, true, true, PG, TQ>(p, grid, s);
    else launch_split_sp<D, C, BITS, true, false, PG, TQ>(p, grid, s);
  } else {
    if (share) launch_split_sp<D, C, BITS, false, true, PG, TQ>(p, grid, s);
    else launch_split_sp<D, C, BITS, false, false, PG, TQ>(p, grid, s);
  }
  return hipGetLastError();
}

}  // namespace loopvq
