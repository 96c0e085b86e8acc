// Kernel parameter blocks and launchers shared between the C ABI layer and
// the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loopvq {

// entries of the per-wave page lists of the workgroup-shared RoPE path (per
// stream): a chunk of the split plan must span at most this many pages
constexpr int DECODE_PAGE_LIST = 128;
// batches of up to this many requests are taken in length order by the quad
// decode (larger ones in index order)
constexpr int DECODE_SORT_MAX = 512;

struct DecodeParams {
  const void* q;              // [B][H_q][D] bf16 or fp32
  const uint8_t* cache;       // [num_pages][H_kv][2][P][R]
  const void* slices;         // slice of the step: [H_kv][2][K][C] fp16
  const float* rope;          // [max_pos][D/16][4][4]
  const int32_t* block_table; // [B][max_pages]
  const int32_t* seq_lens;    // [B] end of each request's coded positions
  const int32_t* seq_lo;      // [B] first coded position (bf16 sink before it), or null for 0
  // TaSQ-coded keys (null unless the TaSQ variant runs): the codes index
  // u = P(w k / sigma); the key is rebuilt as sigma * P^-1(u_hat) / w
  const float* tq_w;          // [H_kv][D] channel weights of this loop step
  const int32_t* tq_perm;     // [H_kv][D/2] pair permutation of this block
  const uint16_t* tq_sigma;   // fp16 scale of this loop step per physical slot (page*P + offset)
  float* part_o;              // [H_kv][n_pairs][n_chunks][D]
  float* part_lse;            // [H_kv][n_pairs][n_chunks], log2 domain
  int B, H_kv, H_q, grp, max_pages, log2P;
  int n_pairs;                // B * grp (request, query head) pairs per KV head
  int n_dg;                   // duos (pairs 2i, 2i+1), or quads (4i .. 4i+3), per KV head; one per wave
  int Lc;                     // positions per chunk (one wave), a multiple of 32 (64 if shared_rope)
  int shared_rope;            // eight waves of a workgroup share a chunk and its RoPE rows
  int quad;                   // a wave serves four query heads of one request (else two pairs)
  int n_chunks;
  int items_per_head;         // n_dg * n_chunks wave work items per KV head
  int wg_per_head;            // ceil(items_per_head / 8): eight waves per workgroup
  int max_seq_len;            // host bound; seq_lens are clamped to it
  float scale_log2;           // sm_scale * log2(e)
};

struct CombineParams {
  const float* part_o;
  const float* part_lse;
  const float* win_o;         // [H_kv][n_pairs][D] bf16-token partials, or null
  const float* win_lse;       // [H_kv][n_pairs], log2 domain
  const int32_t* seq_lens;
  void* out;
  float* lse;
  int B, H_q, grp, n_pairs, n_chunks, Lc, max_seq_len;
};

// attention over the bf16 tokens of each request (sink and recent window)
struct WindowParams {
  const void* q;              // [B][H_q][D] bf16 or fp32
  const uint16_t* kv;         // bf16 pages [num_pages][H_kv][2][8][D], pre-RoPE K and V
  const int32_t* page_table;  // [B][max_pages]: bf16 token u sits in page u/8, slot u%8
  const int32_t* n_sink;      // [B] sink tokens, positions [0, n_sink)
  const int32_t* win_start;   // [B] first position of the recent window
  const int32_t* seq_lens;    // [B] tokens per request; the window is [win_start, seq_len)
  const float* rope;          // the decode kernel's RoPE table
  float* win_o;               // [H_kv][n_pairs][D]
  float* win_lse;             // [H_kv][n_pairs], log2 domain
  int H_kv, H_q, grp, n_pairs, max_pages, max_seq_len;
  float scale_log2;
};

struct EncodeParams {
  const void* xk;             // dense [n_blocks*Tc][n_tok][H_kv][D], or bf16 pages (see src_slot)
  const void* xv;
  const int32_t* src_slot;    // null: dense input; else bf16 pages [step][page][H_kv][2][8][D], token j at
                              // page src_slot[j] / 8, slot src_slot[j] % 8 (xv = xk + 8*D)
  int64_t step_stride;        // elements between consecutive loop steps of the input
  const uint16_t* cb;         // [n_blocks][H_kv][2][K][G] fp16 of the first block
  const float* hsq;           // [n_blocks][H_kv][2][K]
  const int32_t* slot_mapping;
  uint8_t* cache;             // cache of the first block
  int64_t block_stride;
  int n_tok, H_kv, D, c, Tc, K, log2P;
  int per_group;              // one codebook per channel group: units are 32 tokens of one group
  int kv_lo, kv_n;            // code streams kv_lo .. kv_lo + kv_n - 1 of {K, V}
  int units_per_wave;         // units of 32 consecutive (token, group) vectors per wave
  int n_unit_groups;          // ceil(units / (4 * units_per_wave)), the grid's x extent
  int32_t* near_tie;          // device counter the near-tie count is added to, or null
};

// TaSQ key transform: u = P(w k / sigma) and the fp16 sigma of every token
struct TasqParams {
  const void* xk;             // [n_steps][n_tok][H][D] pre-RoPE keys, bf16 or fp32
  const float* w;             // [T][H][D] channel weights
  const int32_t* perm;        // [T/Tc][H][D/2] pair permutations
  const int32_t* slot_mapping;  // [n_tok] physical slot of each token
  uint16_t* sigma;            // fp16 scale of loop step t, slot s at t*sigma_stride + s
  int64_t sigma_stride;
  float* u;                   // [n_steps][n_tok][H][D] fp32
  int n_tok, H, D, Tc, first_step;
};

// codebook update of one Lloyd iteration (the codes come from the encoder)
struct KmeansParams {
  const void* xk;             // [n_blocks*Tc][n_tok][H_kv][D], bf16 or fp32
  const void* xv;
  const int32_t* slot_mapping;
  const uint8_t* cache;       // index cache of the first block
  int64_t block_stride;
  const uint16_t* cb;         // [n_blocks][H_kv][2][K][G] fp16 codebooks that assigned the codes
  uint16_t* cb_out;           // updated codebooks, same layout
  double* err;                // [n_blocks][H_kv][2][2]: sum ||z - e||^2, sum ||z||^2, or null
  double* gsum;               // workspace: per stream [K][G] sums, [K] counts, 2 error sums
  int n_tok, H_kv, D, c, Tc, K, bits, log2P;
  int tok_per_wg;
};

hipError_t launch_decode_split(int D, int C, int bits, bool qf32, const DecodeParams& p, int grid,
                               hipStream_t s);
hipError_t launch_decode_split_pg(int D, int C, int bits, bool qf32, const DecodeParams& p, int grid,
                                  hipStream_t s);
hipError_t launch_decode_split_tq(int D, int C, int bits, bool qf32, const DecodeParams& p, int grid,
                                  hipStream_t s);
hipError_t launch_decode_combine(int D, bool out_bf16, const CombineParams& p, hipStream_t s);
hipError_t launch_decode_window(int D, bool qf32, const WindowParams& p, int B, hipStream_t s);
hipError_t launch_encode(int G, bool xf32, int bits, const EncodeParams& p, int n_blocks, hipStream_t s);
hipError_t launch_tasq_transform(bool xf32, const TasqParams& p, int n_steps, hipStream_t s);
hipError_t launch_kmeans_update(bool xf32, const KmeansParams& p, int n_blocks, hipStream_t s);
hipError_t launch_build_slices(const uint16_t* cb, uint16_t* slices, float* hsq, int n_blocks, int H_kv,
                               int K, int c, int Tc, hipStream_t s);

}  // namespace loopvq
