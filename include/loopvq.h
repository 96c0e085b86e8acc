/*
 * loopvq.h - C ABI of the LoopVQ encoder and quantised decode-attention
 * library for AMD Instinct MI355X (gfx950).
 *
 * LoopVQ ("LoopVQ: Sub 1-bit KV Cache Quantization for Looped Transformers",
 * hub.valency.io/works/W_7srt5hed_v1) quantises the KV cache of a looped
 * transformer along the loop axis: T loop steps are cut into blocks of Tc
 * consecutive steps, and one b-bit code covers c channels at each of the Tc
 * steps of a block (a coupled vector of G = c*Tc elements, section "Loop-axis vector
 * quantization", eq. (4)).  Loop step beta*Tc + m + 1 reads the shared code through its own
 * slice of the codebook entry, coordinates i*Tc + m for i < c (eq. (5) and
 * section "System implementation").  Keys are coded before RoPE, and the
 * decode kernel applies RoPE to every rebuilt key (section "Preliminaries"; appendix "Optimizing pre-RoPE vector
 * quantization serving efficiency").
 *
 * Conventions
 *   - Every pointer is a device pointer unless marked [host].  The caller owns
 *     every buffer; the library allocates and frees no memory and keeps no
 *     state between calls, so calls on different streams are independent.
 *   - All device work is enqueued on the given stream; no call synchronises.
 *   - Every argument is validated on the host before anything is launched;
 *     a call that returns an error has enqueued nothing.
 *   - Functions return LOOPVQ_OK (0) or a negative status; no C++ exception
 *     crosses this interface.
 *   - Device faults (for example a block-table entry outside the index cache)
 *     are undefined behaviour and surface as HIP errors on the caller's next
 *     synchronisation.
 *
 * Data layouts
 *   codebook  cb     [n_blocks][H_kv][2][K][G] fp16, entry coordinate
 *                    u = i*Tc + m (channel-major, loop-minor), index 1 = K|V.
 *                    With per_group: [n_blocks][H_kv][2][D/c][K][G], one
 *                    codebook per channel group (the pages' B_{beta,l,h,g},
 *                    section "Loop-axis vector quantization").
 *   slices           [T][H_kv][2][K][c] fp16: slice of loop step t (0-based
 *                    here) holds coordinates i*Tc + (t mod Tc) of each entry
 *                    (per_group: [T][H_kv][2][D/c][K][c]).
 *   hsq              [n_blocks][H_kv][2][K] fp32: 0.5*||e||^2 of each entry
 *                    (per_group: [n_blocks][H_kv][2][D/c][K]).
 *   index cache      one cache per block beta: [num_pages][H_kv][2][P][R]
 *                    bytes, R = (D/c)*bits/8 bytes per row.  Page p holds the
 *                    rows of tokens p*P .. p*P+P-1 of whichever request maps
 *                    a logical page to it through its block table.  One page
 *                    (H_kv*2*P*R bytes) must be smaller than 4 GiB, else
 *                    every entry point returns LOOPVQ_ERR_UNSUPPORTED.
 *   row order        A row stores the n = D/c codes of one token in the
 *                    "RoPE-pair interleaved" slot order: with h = n/2 and
 *                    q = n/8, slot s = i*2q + r (i < 4, r < 2q) holds group
 *                    g(s) = i*q + r when r < q and h + i*q + (r - q) otherwise,
 *                    so the groups {g, g + h} whose channels RoPE rotates
 *                    together sit side by side.  8-bit: slot s is byte s.
 *                    4-bit: slot s is the low nibble of byte s/2 when s is
 *                    even, the high nibble when odd.
 *   rope table       fp32, positions interleaved in groups of 4 (see loopvq_rope_table).
 *   q, out           [B][H_q][D], query head j reads KV head j / (H_q/H_kv).
 */
#ifndef LOOPVQ_H
#define LOOPVQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  LOOPVQ_OK = 0,
  LOOPVQ_ERR_INVALID_ARG = -1,      /* null pointer, inconsistent sizes, bad t, ...     */
  LOOPVQ_ERR_UNSUPPORTED = -2,      /* valid but not compiled: bits, c, D, dtype, ...   */
  LOOPVQ_ERR_WORKSPACE = -3,        /* decode workspace smaller than required           */
  LOOPVQ_ERR_HIP = -4,              /* a HIP launch or runtime call failed              */
  LOOPVQ_ERR_SCRATCH = -5           /* batch needs more than the fixed device scratch   */
};

enum { LOOPVQ_DTYPE_F32 = 0, LOOPVQ_DTYPE_BF16 = 1 };

typedef struct loopvq_dims {
  int32_t D;          /* head dimension: 64 or 128                                      */
  int32_t c;          /* channels per loop step covered by one code: 2, 4 or 8 (16 with
                         Tc = 1: G channels of one step, for the encoder and k-means only) */
  int32_t Tc;         /* loop steps per block (one code serves Tc steps); Tc | T        */
  int32_t T;          /* loop steps                                                     */
  int32_t bits;       /* code width: 4 or 8                                             */
  int32_t K;          /* codebook entries, must equal 1 << bits                         */
  int32_t H_kv;       /* KV heads                                                       */
  int32_t H_q;        /* query heads, a multiple of H_kv                                */
  int32_t page_size;  /* tokens per page P: a power of two in [8, 1024]                 */
  int32_t x_dtype;    /* encoder input K/V: LOOPVQ_DTYPE_F32 or LOOPVQ_DTYPE_BF16        */
  int32_t io_dtype;   /* decode query and output: LOOPVQ_DTYPE_F32 or LOOPVQ_DTYPE_BF16  */
  int32_t per_group;  /* 0: one codebook per (block, KV head, K|V), shared by the D/c
                         channel groups; 1: one codebook per channel group as well
                         (8-bit codes only)                                             */
} loopvq_dims;
/* Supported shapes: D in {64, 128}; D/c a multiple of 8 (of 16 for the encoder
 * with 4-bit codes); G = c*Tc in {8, 16, 32} (G = 8 only with fp32 encoder
 * input); 4-bit codes only with K = 16 and 8-bit only with K = 256. */

/* Human-readable text of a status code.  Never NULL. */
const char* loopvq_status_string(int status);

/* Bytes of one index row, (D/c)*bits/8, or a negative status. */
int loopvq_row_bytes(const loopvq_dims* dims);

/*
 * Cut the per-loop-step codebook slices once at load time, and compute
 * hsq = 0.5*||e||^2 of every entry (in fp64, rounded to fp32) for the encoder.
 * [LoopVQ paper, section "System implementation": the slice B_t holds
 * coordinate i*Tc + m of every entry, cut once when the model is loaded.]
 *   n_blocks = T / Tc codebooks per (KV head, K|V).
 *   cb      [n_blocks][H_kv][2][K][G] fp16 (input)
 *   slices  [T][H_kv][2][K][c] fp16      (output)
 *   hsq     [n_blocks][H_kv][2][K] fp32  (output, may be NULL)
 */
int loopvq_build_codebook_slices(const loopvq_dims* dims, const void* cb,
                                 void* slices, float* hsq, hipStream_t stream);

/*
 * Host-side RoPE coefficient table in the layout the decode kernel streams.
 * The table is padded to 16*ceil(max_pos/16) positions (the decode kernel
 * reads 16 positions per step); for position p = 4g + n, chunk j < D/16 and
 * lane quarter i < 4, the four floats at (((g*(D/16) + j)*4 + i)*4 + n)*4 are
 *     cos(p*theta_f), sin(p*theta_f), cos(p*theta_{f+1}), sin(p*theta_{f+1})
 * with f = i*(D/8) + 2*j and theta_f = base^(-2f/D), computed in fp64 and
 * rounded to fp32.  [LoopVQ paper, appendix "Optimizing pre-RoPE vector
 * quantization serving efficiency": the kernel reads cos/sin from a table
 * precomputed for all positions instead of evaluating transcendentals.]
 *   table [host] must hold loopvq_rope_table_floats(max_pos, D) floats.  The
 *   caller copies it to the device once.
 */
int loopvq_rope_table(int32_t max_pos, int32_t D, double base, float* table);

/* Floats of the RoPE table for max_pos positions (0 on invalid arguments). */
size_t loopvq_rope_table_floats(int32_t max_pos, int32_t D);

/*
 * Encode blocks of pre-RoPE keys and values into the paged index caches.
 * For every token j, KV head h, x in {K, V}, block beta and group g < D/c,
 * the coupled vector z[i*Tc + m] = x^(beta*Tc+m+1)[j][h][g*c + i] (eq. 4)
 * is replaced by the index of its nearest codebook entry in squared L2
 * distance, ties to the lowest index (eq. 2), and written to slot g's place
 * in the row of token j.  [LoopVQ paper, section "System implementation",
 * encoding: distances to all entries as a matrix product, then the nearest
 * entry.]
 *   n_tok         tokens in this call (n_tok >= 0; 0 is a no-op).
 *   n_blocks      blocks encoded, 1 <= n_blocks <= T/Tc; block beta of x is
 *                 loop steps beta*Tc .. beta*Tc+Tc-1 of the input.
 *   xk, xv        [n_blocks*Tc][n_tok][H_kv][D], dtype dims->x_dtype.
 *   cb, hsq       codebooks and 0.5*||e||^2 of blocks first_block ..
 *                 first_block+n_blocks-1, layouts as above (hsq from
 *                 loopvq_build_codebook_slices).
 *   slot_mapping  [n_tok] int32 physical slot page*P + offset of each token,
 *                 in [0, num_pages*P) (device data, not checked: a slot
 *                 outside the cache writes outside it).
 *   index_cache   cache of block first_block; block beta's cache starts at
 *                 index_cache + (beta - first_block)*block_stride_bytes.
 *   near_tie_count  NULL, or one device int32 (4-byte aligned) to which the
 *                 call adds the number of coupled vectors it coded whose two
 *                 smallest distances lie within 1e-6*(||z||^2 + ||e_a||^2) of
 *                 each other (e_a the chosen entry), as judged on the fp32
 *                 scores the encoder computes; exact ties (duplicate entries)
 *                 always count.  The caller zeroes it.  NULL runs the plain
 *                 encoder, which does no near-tie work; a count costs a
 *                 second scoring pass over the codebook.
 * Distances are evaluated as ||z||^2 - 2 z.e + ||e||^2 with fp16 inputs and
 * fp32 accumulation (bf16 inputs convert exactly to fp16 inside fp16's normal
 * range; fp32 inputs are split into two fp16 terms), so the index can differ
 * from an exact evaluation only where two distances lie within fp32 rounding
 * of each other.  Entries whose fp16 values are identical score identically,
 * and the lowest of their indices is the one written.
 */
int loopvq_encode(const loopvq_dims* dims, int32_t n_tok, int32_t first_block,
                  int32_t n_blocks, const void* xk, const void* xv,
                  const void* cb, const float* hsq, const int32_t* slot_mapping,
                  uint8_t* index_cache, int64_t block_stride_bytes,
                  int32_t* near_tie_count, hipStream_t stream);

/*
 * Decode-time page encoding: code tokens held in bf16 pages (the recent
 * window) into the paged index caches, for every loop step of the given
 * blocks at once.  [LoopVQ paper, section "System implementation",
 * encoding: during decoding each new token's keys and values go to the bf16
 * window, where all its loop steps are available after the forward pass, and
 * every delta generated tokens the oldest window page is coded across all
 * layers and loop steps into one quantised page.]  The arithmetic and the
 * result are those of loopvq_encode on the same values.
 *   n_tok         tokens to code (0 is a no-op).
 *   kv_pages      bf16 page pool of loop step first_block*Tc:
 *                 [num_pages][H_kv][2][8][D] (index 0 the pre-RoPE key, 1 the
 *                 value), 16-byte aligned; loop step first_block*Tc + s is the
 *                 pool at kv_pages + s*step_stride elements.
 *   step_stride   elements between the pools of consecutive loop steps
 *                 (a multiple of 8; may be 0 only when n_blocks*Tc == 1).
 *   src_slot      [n_tok] int32: page*8 + slot of each token in the pools.
 *   cb, hsq, slot_mapping, index_cache, block_stride_bytes, first_block,
 *   n_blocks      as for loopvq_encode.
 * Requires dims->x_dtype == LOOPVQ_DTYPE_BF16 (else LOOPVQ_ERR_UNSUPPORTED).
 */
int loopvq_encode_pages(const loopvq_dims* dims, int32_t n_tok, int32_t first_block,
                        int32_t n_blocks, const void* kv_pages, int64_t step_stride,
                        const int32_t* src_slot, const void* cb, const float* hsq,
                        const int32_t* slot_mapping, uint8_t* index_cache,
                        int64_t block_stride_bytes, hipStream_t stream);

/* Workspace bytes that loopvq_decode_attn and loopvq_decode_attn_window need
 * for this batch shape. */
size_t loopvq_decode_workspace_bytes(const loopvq_dims* dims, int32_t B,
                                     int32_t max_seq_len);

/*
 * Quantised decode attention of B requests at loop step t (1-based).
 * [LoopVQ paper, section "System implementation", attention: at loop step
 * t each index is looked up in B_t to rebuild K, RoPE is applied, and the
 * tokens are spread over workgroups; joining their partial outputs by
 * log-sum-exp gives the same softmax as one pass over all tokens.]
 *   t             loop step, 1 <= t <= T; reads block (t-1)/Tc, slice t-1.
 *   q             [B][H_q][D] queries already rotated at their own position.
 *                 bf16 queries enter the matrix cores as fp16 values, so
 *                 every |q_i| must stay below 65504 (fp16's largest finite
 *                 value; larger values become infinite scores); magnitudes
 *                 below 2^-14 are rounded to fp16 subnormals (an absolute
 *                 error below 2^-25).  fp32 queries are carried as two fp16
 *                 terms and need |q_i| below 65504 as well.  (With a GQA
 *                 group that is a multiple of four, bf16 queries and pages
 *                 of 16 or more positions, the scores are taken in fp32
 *                 and these limits do not bind; callers should not rely on
 *                 that.)
 *   index_cache   the cache of block (t-1)/Tc.
 *   slices        [T][H_kv][2][K][c] fp16 from loopvq_build_codebook_slices.
 *   rope_table    device copy of loopvq_rope_table(max_pos, D, base).
 *   block_table   [B][max_pages] int32 physical page of each logical page,
 *                 in [0, num_pages) for every logical page a request's
 *                 seq_len covers (device data, not checked).
 *   seq_lens      [B] int32 cached tokens per request, 0 <= seq_lens[b] <=
 *                 max_seq_len, and max_seq_len <= max_pos, and
 *                 max_seq_len <= max_pages*P.  Token j of a request sits at
 *                 RoPE position j.
 *   sm_scale      softmax scale; <= 0 selects 1/sqrt(D).
 *   out           [B][H_q][D] attention output (dims->io_dtype).  A request
 *                 with no cached tokens gets zeros.
 *   lse           [B][H_q] fp32 natural-log sum of exp(scores), or NULL;
 *                 -inf for a request with no tokens.
 *   workspace     at least loopvq_decode_workspace_bytes(dims, B, max_seq_len)
 *                 bytes of device memory, 256-byte aligned; contents on entry
 *                 are ignored.
 */
int loopvq_decode_attn(const loopvq_dims* dims, int32_t t, int32_t B,
                       const void* q, const uint8_t* index_cache,
                       const void* slices, const float* rope_table,
                       int32_t max_pos, const int32_t* block_table,
                       int32_t max_pages, const int32_t* seq_lens,
                       int32_t max_seq_len, float sm_scale, void* out,
                       float* lse, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * The two phases of loopvq_decode_attn as separate calls, for callers that
 * time or schedule them apart.  loopvq_decode_split runs the split-K pass and
 * leaves per-split partial outputs and log-sum-exps in the workspace;
 * loopvq_decode_combine merges them into out and lse.  Both must be given the
 * same dims, B, seq_lens, max_seq_len and workspace, on the same stream (or
 * with the caller ordering them).  Arguments mean what they mean for
 * loopvq_decode_attn.  [LoopVQ paper, section "System implementation":
 * split partial outputs combined through the logsumexp of their scores.]
 */
int loopvq_decode_split(const loopvq_dims* dims, int32_t t, int32_t B, const void* q,
                        const uint8_t* index_cache, const void* slices,
                        const float* rope_table, int32_t max_pos,
                        const int32_t* block_table, int32_t max_pages,
                        const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);
int loopvq_decode_combine(const loopvq_dims* dims, int32_t B, const int32_t* seq_lens,
                          int32_t max_seq_len, void* out, float* lse,
                          const void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Bytes of the fixed device scratch of loopvq_decode_attn_noalloc (8 MiB). */
#define LOOPVQ_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * loopvq_decode_attn for callers that cannot allocate device memory (code
 * under stream or graph capture, serving loops and harnesses that forbid
 * hipMalloc): the same kernels and the same result bit for bit, with the
 * split partials kept in a fixed device array of the library instead of a
 * caller workspace.  The call allocates nothing.
 *   Limit: the batch's loopvq_decode_workspace_bytes(dims, B, max_seq_len)
 *          must not exceed LOOPVQ_NOALLOC_SCRATCH_BYTES, else the call returns
 *          LOOPVQ_ERR_SCRATCH and enqueues nothing (for example 16 requests of
 *          32K tokens and 16 heads need 2.2 MiB).
 *   Scope: each GPU holds one copy of the array, from the first call on that
 *          device (the call that looks its address up, with the device
 *          current) until the process ends.  Every call on one GPU uses that
 *          GPU's copy: calls on one GPU whose work may overlap (other streams,
 *          other host threads) race on it and must be ordered by the caller.
 *          Nothing in it needs to start at zero.
 *   stream must belong to the current device.  Other arguments as for
 *   loopvq_decode_attn.
 */
int loopvq_decode_attn_noalloc(const loopvq_dims* dims, int32_t t, int32_t B,
                               const void* q, const uint8_t* index_cache,
                               const void* slices, const float* rope_table,
                               int32_t max_pos, const int32_t* block_table,
                               int32_t max_pages, const int32_t* seq_lens,
                               int32_t max_seq_len, float sm_scale, void* out,
                               float* lse, hipStream_t stream);

/*
 * The bf16 pages of a request: its attention sink and its recent window.
 * [LoopVQ paper, section "System implementation", cache layout: the first
 * n_s tokens and the most recent tokens of a request stay in bf16, in pages of
 * 8 tokens, and every other token is coded; the window is coded a page at a
 * time as it moves on, so its keys are kept before RoPE.]
 *   kv          bf16 pages of the loop step being attended:
 *               [num_pages][H_kv][2][8][D], index 0 the pre-RoPE key, 1 the
 *               value; 16-byte aligned.
 *   page_table  [B][max_pages] int32.  Number the bf16 tokens of request b
 *               u = 0, 1, ...: first its sink positions 0 .. n_sink-1, then
 *               its window positions win_start .. seq_len-1.  Token u sits in
 *               page page_table[b][u / 8], slot u % 8.
 *   n_sink      [B] int32 sink tokens of each request (positions [0, n_sink)).
 *   win_start   [B] int32 first position of the recent window; positions
 *               [win_start, seq_len) are bf16.
 * Requires 0 <= n_sink[b] <= win_start[b] <= seq_lens[b] and
 * ceil((n_sink + seq_len - win_start) / 8) <= max_pages (device values, not
 * checked on the host; out-of-order values are clamped into that order).
 */
typedef struct loopvq_bf16_window {
  const void* kv;
  const int32_t* page_table;
  int32_t max_pages;
  const int32_t* n_sink;
  const int32_t* win_start;
} loopvq_bf16_window;

/*
 * Decode attention at loop step t over a cache that mixes bf16 pages (sink
 * and recent window) with coded pages.  [LoopVQ paper, section "System
 * implementation", attention: the unquantised pages and the coded pages are
 * attended by separate kernels, and joining their partials by log-sum-exp
 * gives a single softmax over every cached token.]
 * Positions [n_sink, win_start) of request b are read as codes through
 * block_table, exactly as loopvq_decode_attn reads positions [0, seq_len);
 * block-table entries of pages that hold no coded position are never read.
 * The other positions come from the bf16 pages; every key is rotated at its
 * own position.  seq_lens holds the full length of each request.  Other
 * arguments as for loopvq_decode_attn; workspace_bytes must be at least
 * loopvq_decode_workspace_bytes(dims, B, max_seq_len).
 */
int loopvq_decode_attn_window(const loopvq_dims* dims, int32_t t, int32_t B,
                              const void* q, const uint8_t* index_cache,
                              const void* slices, const float* rope_table,
                              int32_t max_pos, const int32_t* block_table,
                              int32_t max_pages, const int32_t* seq_lens,
                              int32_t max_seq_len,
                              const loopvq_bf16_window* window, float sm_scale,
                              void* out, float* lse, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * TaSQ-coded keys (TaSQ+LoopVQ).  [LoopVQ paper, appendix "Orthogonal
 * application with TaSQ": "Formulation" (eqs. (10)-(11)), "Grouping under
 * loop coupling", "Calibration and bitwidth".]  Before coupling, the pre-RoPE
 * key of loop step t, head h and token j is mapped to
 *     u = P_{beta,h}(w_{t,h} (.) k / sigma_{t,j}),
 * sigma_{t,j} being the root mean square of w_{t,h} (.) k over all heads and
 * channels of token j at step t, kept in fp16 (round to nearest even; a
 * token whose fp16 sigma is 0 gets u = 0).  P moves RoPE pairs as units and
 * keeps each pair inside one code: u channel 2p holds key channel perm[p] and
 * u channel 2p+1 holds perm[p] + D/2.  Keys are coded from u (values as
 * usual), and decode rebuilds k_hat = sigma * P^-1(u_hat) / w before RoPE.
 *   w             [T][H_kv][D] fp32 channel weights, positive; |q_i / w_i|
 *                 must stay inside fp16's range.
 *   perm          [T/Tc][H_kv][D/2] int32, each row a permutation of
 *                 0 .. D/2-1 (other values give unspecified results).
 *   sigma         fp16 scales: loop step t (0-based), physical slot s
 *                 (page*P + offset) at sigma[t*sigma_stride + s].  Written by
 *                 loopvq_encode_tasq, read by loopvq_decode_attn_tasq.
 *   sigma_stride  elements between the arrays of consecutive loop steps
 *                 (even; > 0 when T > 1).  sigma is 4-byte aligned.
 * TaSQ-coded keys need 8-bit codes, one codebook per (block, head, K|V)
 * (per_group = 0) and H_kv*D <= 10922; other shapes return
 * LOOPVQ_ERR_UNSUPPORTED.  The K codebooks are codebooks of u.
 */
typedef struct loopvq_tasq {
  const float* w;
  const int32_t* perm;
  uint16_t* sigma;
  int64_t sigma_stride;
} loopvq_tasq;

/* Workspace bytes of loopvq_encode_tasq (u of every coded loop step, fp32). */
size_t loopvq_encode_tasq_workspace_bytes(const loopvq_dims* dims, int32_t n_tok,
                                          int32_t n_blocks);

/*
 * loopvq_encode with TaSQ-coded keys: computes sigma (stored at each token's
 * slot for every coded loop step) and u, then codes u as the keys and xv as
 * the values.  Arguments as for loopvq_encode; xk holds the pre-RoPE keys.
 * xk and tasq->w must be 16-byte aligned.  workspace: at least
 * loopvq_encode_tasq_workspace_bytes(dims, n_tok, n_blocks) bytes, 256-byte
 * aligned.  The key codes differ from an exact
 * evaluation only where two distances lie within fp32 rounding of each other
 * (u is formed in fp64 and rounded once to fp32), and sigma only where the
 * exact RMS lies within fp64 rounding of an fp16 rounding midpoint.
 */
int loopvq_encode_tasq(const loopvq_dims* dims, int32_t n_tok, int32_t first_block,
                       int32_t n_blocks, const void* xk, const void* xv,
                       const loopvq_tasq* tasq, const void* cb, const float* hsq,
                       const int32_t* slot_mapping, uint8_t* index_cache,
                       int64_t block_stride_bytes, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * Decode attention at loop step t over TaSQ-coded keys: reads w of step t,
 * perm of block (t-1)/Tc and the sigma array of step t.  With window non-NULL
 * the bf16 sink and recent window are attended as in loopvq_decode_attn_window
 * (their keys are plain pre-RoPE keys); with window NULL this is
 * loopvq_decode_attn.  Other arguments as for those calls.
 */
int loopvq_decode_attn_tasq(const loopvq_dims* dims, int32_t t, int32_t B,
                            const void* q, const uint8_t* index_cache,
                            const void* slices, const float* rope_table,
                            int32_t max_pos, const int32_t* block_table,
                            int32_t max_pages, const int32_t* seq_lens,
                            int32_t max_seq_len, const loopvq_tasq* tasq,
                            const loopvq_bf16_window* window, float sm_scale,
                            void* out, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * Plain k-means on the coupled vectors of a layer, one Lloyd iteration per
 * pair of calls: loopvq_encode assigns every coupled vector to its nearest
 * entry (the codes it writes), then loopvq_kmeans_update moves each entry to
 * the mean of the vectors coded with it.  [LoopVQ paper, section "Redundancy
 * along the loop axis", Fig. 2c: unweighted k-means under the loop-axis
 * grouping and under G channels of one step (c = G, Tc = 1 on the steps laid
 * end to end as tokens), same bit width and number of codebooks.]
 * The means are exact fp64 sums of the vectors divided by their count,
 * rounded to fp16 (round to nearest even); an entry no vector uses keeps its
 * value.  Arguments as for loopvq_encode (the same xk, xv, slot_mapping and
 * index cache the assigning call used), plus:
 *   cb        codebooks that assigned the codes (of blocks first_block ..),
 *   cb_out    the updated codebooks, same layout (may not alias cb),
 *   err       [n_blocks][H_kv][2][2] fp64 or NULL: sum over the coupled
 *             vectors of ||z - e_code||^2 (e from cb) and of ||z||^2,
 *   workspace loopvq_kmeans_workspace_bytes(dims, n_blocks) bytes, 256-byte
 *             aligned.
 * Requires per_group = 0.
 */
size_t loopvq_kmeans_workspace_bytes(const loopvq_dims* dims, int32_t n_blocks);
int loopvq_kmeans_update(const loopvq_dims* dims, int32_t n_tok, int32_t first_block,
                         int32_t n_blocks, const void* xk, const void* xv,
                         const int32_t* slot_mapping, const uint8_t* index_cache,
                         int64_t block_stride_bytes, const void* cb, void* cb_out,
                         double* err, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LOOPVQ_H */
