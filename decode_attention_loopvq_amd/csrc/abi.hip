// C ABI of the LoopVQ library: host-side validation, work planning and launches.
// Every check runs before anything is enqueued, so a call that fails has
// launched nothing.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "loopvq.h"

using namespace loopvq;

namespace {

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int x) { int r = 0; while ((1 << r) < x) ++r; return r; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_dims(const loopvq_dims* d) {
  if (d == nullptr) return LOOPVQ_ERR_INVALID_ARG;
  if (d->D <= 0 || d->c <= 0 || d->Tc <= 0 || d->T <= 0 || d->H_kv <= 0 || d->H_q <= 0)
    return LOOPVQ_ERR_INVALID_ARG;
  if (d->D % d->c != 0 || d->T % d->Tc != 0 || d->H_q % d->H_kv != 0) return LOOPVQ_ERR_INVALID_ARG;
  if (d->bits <= 0 || d->bits > 16 || d->K != (1 << d->bits)) return LOOPVQ_ERR_INVALID_ARG;
  if (!is_pow2(d->page_size) || d->page_size < 8 || d->page_size > 1024) return LOOPVQ_ERR_INVALID_ARG;
  if ((d->x_dtype != LOOPVQ_DTYPE_F32 && d->x_dtype != LOOPVQ_DTYPE_BF16) ||
      (d->io_dtype != LOOPVQ_DTYPE_F32 && d->io_dtype != LOOPVQ_DTYPE_BF16))
    return LOOPVQ_ERR_INVALID_ARG;
  if (d->bits != 4 && d->bits != 8) return LOOPVQ_ERR_UNSUPPORTED;
  if (d->D != 64 && d->D != 128) return LOOPVQ_ERR_UNSUPPORTED;
  // c = 16 (with Tc = 1) is encoder-only: G channels of one step, the baseline grouping
  if (d->c != 2 && d->c != 4 && d->c != 8 && d->c != 16) return LOOPVQ_ERR_UNSUPPORTED;
  if (d->c == 16 && d->Tc != 1) return LOOPVQ_ERR_UNSUPPORTED;
  if ((d->D / d->c) % 8 != 0) return LOOPVQ_ERR_UNSUPPORTED;
  const int G = d->c * d->Tc;
  if (G != 8 && G != 16 && G != 32) return LOOPVQ_ERR_UNSUPPORTED;
  if (G == 8 && d->x_dtype != LOOPVQ_DTYPE_F32) return LOOPVQ_ERR_UNSUPPORTED;
  if (d->per_group != 0 && d->per_group != 1) return LOOPVQ_ERR_INVALID_ARG;
  if (d->per_group && d->bits != 8) return LOOPVQ_ERR_UNSUPPORTED;
  // the kernels take the bytes of one index-cache page as a 32-bit value
  const long long row_bytes = (long long)(d->D / d->c) * d->bits / 8;
  if ((long long)d->H_kv * 2 * d->page_size * row_bytes > 0xffffffffLL) return LOOPVQ_ERR_UNSUPPORTED;
  return LOOPVQ_OK;
}

// codebooks per (block, KV head, K|V): one, or one per channel group
int n_codebook_groups(const loopvq_dims* d) { return d->per_group ? d->D / d->c : 1; }

struct DecodePlan {
  int grp, n_pairs, NT, n_dg, Lc, n_chunks, items_per_head, wg_per_head, grid, shared_rope, quad;
  size_t n_part, bytes_o, bytes_lse;
  size_t bytes_wo, bytes_wl;   // bf16-token partials: one per (KV head, pair)
  size_t total() const { return bytes_o + bytes_lse + bytes_wo + bytes_wl; }
};

// A wave serves one duo of (request, query head) pairs (2i, 2i+1) over one
// chunk of Lc positions, NT = 16 consecutive positions per step; the eight
// waves of a workgroup share a KV head (and its LDS slices).
DecodePlan plan_decode(const loopvq_dims* d, int B, int max_seq_len) {
  DecodePlan pl{};
  pl.grp = d->H_q / d->H_kv;
  pl.n_pairs = B * pl.grp;
  pl.NT = 16;
  // quads (four query heads of one request per wave) when the GQA group is a
  // multiple of four, with bf16 queries, pages of 16 or more positions and one
  // codebook per (block, head, K|V); else duos of two pairs
  pl.quad = pl.grp % 4 == 0 && d->io_dtype == LOOPVQ_DTYPE_BF16 && d->page_size >= 16 && !d->per_group;
  pl.n_dg = std::max(1, (pl.n_pairs + (pl.quad ? 3 : 1)) / (pl.quad ? 4 : 2));
  const long long len = std::max(max_seq_len, 1);
  // workgroup-shared RoPE rows: the eight waves of a workgroup must hold eight
  // duos of one chunk (pages of >= 16 positions, bf16 queries)
  pl.shared_rope = pl.n_dg % 8 == 0 && d->page_size >= 16 && d->io_dtype == LOOPVQ_DTYPE_BF16;
  const long long work = (long long)d->H_kv * pl.n_dg * len;
  const long long step2 = (pl.shared_rope ? 4LL : 2LL) * pl.NT;   // steps per loop iteration
  // about 2048 waves (8 per CU) over the whole call.  Quads about 16384, in
  // chunks of at least 512 positions: their workgroups take (group, chunk)
  // items in order of decreasing work, so on ragged batches the many short
  // items of the later rounds even out the CUs' loads
  const long long waves = pl.quad ? 16384 : 2048;
  long long Lc = (work + waves - 1) / waves;
  if (pl.quad) Lc = std::max(Lc, 512LL);
  Lc = (Lc + step2 - 1) / step2 * step2;
  // shared rows keep each chunk's page ids in a DECODE_PAGE_LIST-entry list
  // per stream.  Chunks start at multiples of Lc, a multiple of step2: when
  // the page size divides step2 they start on a page boundary and span at most
  // Lc / P pages; otherwise at most Lc / P + 1
  if (pl.shared_rope) {
    const long long pages = step2 % d->page_size == 0 ? DECODE_PAGE_LIST : DECODE_PAGE_LIST - 1;
    Lc = std::min(Lc, (pages * d->page_size) / step2 * step2);
  }
  Lc = std::max(Lc, step2);
  Lc = std::min(Lc, (len + step2 - 1) / step2 * step2);
  pl.Lc = (int)Lc;
  pl.n_chunks = (int)((len + pl.Lc - 1) / pl.Lc);
  pl.items_per_head = pl.n_dg * pl.n_chunks;
  pl.wg_per_head = (pl.items_per_head + 7) / 8;   // eight waves per workgroup
  pl.grid = d->H_kv * pl.wg_per_head;
  pl.n_part = (size_t)d->H_kv * std::max(pl.n_pairs, 1) * pl.n_chunks;
  pl.bytes_o = align256(pl.n_part * d->D * sizeof(float));
  pl.bytes_lse = align256(pl.n_part * sizeof(float));
  pl.bytes_wo = align256((size_t)d->H_kv * std::max(pl.n_pairs, 1) * d->D * sizeof(float));
  pl.bytes_wl = align256((size_t)d->H_kv * std::max(pl.n_pairs, 1) * sizeof(float));
  return pl;
}

bool decode_supported(int D, int c, int bits) {
  if (D == 128) return c == 2 || c == 4 || c == 8;
  return (c == 2 || c == 4) || (c == 8 && bits == 8);
}

int hip_status(hipError_t e) { return e == hipSuccess ? LOOPVQ_OK : LOOPVQ_ERR_HIP; }

// TaSQ-coded keys: 8-bit codes with one codebook per (block, head, K|V), the
// shapes the TaSQ decode kernels are compiled for
int check_tasq(const loopvq_dims* d, const loopvq_tasq* tq) {
  int st = check_dims(d);
  if (st != LOOPVQ_OK) return st;
  if (tq == nullptr || !tq->w || !tq->perm || !tq->sigma || tq->sigma_stride < 0) return LOOPVQ_ERR_INVALID_ARG;
  // decode reads the sigma of two adjacent slots as one 4-byte word
  if (((uintptr_t)tq->sigma & 3) != 0 || (tq->sigma_stride & 1) != 0) return LOOPVQ_ERR_INVALID_ARG;
  if (d->T > 1 && tq->sigma_stride == 0) return LOOPVQ_ERR_INVALID_ARG;
  if (d->bits != 8 || d->per_group) return LOOPVQ_ERR_UNSUPPORTED;
  // the transform keeps the inverse pair permutation and one token's u row in 64 KiB of LDS
  if ((long long)d->H_kv * d->D * 6 > 65536) return LOOPVQ_ERR_UNSUPPORTED;
  return LOOPVQ_OK;
}

}  // namespace

extern "C" {

const char* loopvq_status_string(int status) {
  switch (status) {
    case LOOPVQ_OK: return "ok";
    case LOOPVQ_ERR_INVALID_ARG: return "invalid argument";
    case LOOPVQ_ERR_UNSUPPORTED: return "unsupported shape, code width or dtype";
    case LOOPVQ_ERR_WORKSPACE: return "workspace too small";
    case LOOPVQ_ERR_HIP: return "HIP runtime or launch error";
    case LOOPVQ_ERR_SCRATCH: return "batch needs more than the fixed device scratch of the no-allocation decode";
    default: return "unknown status";
  }
}

int loopvq_row_bytes(const loopvq_dims* dims) {
  const int st = check_dims(dims);
  if (st != LOOPVQ_OK) return st;
  return dims->D / dims->c * dims->bits / 8;
}

int loopvq_build_codebook_slices(const loopvq_dims* dims, const void* cb, void* slices, float* hsq,
                                 hipStream_t stream) {
  int st = check_dims(dims);
  if (st != LOOPVQ_OK) return st;
  if (cb == nullptr || slices == nullptr) return LOOPVQ_ERR_INVALID_ARG;
  // one codebook per group: the groups' entries follow one another, so the
  // slices are those of a codebook of n*K entries
  return hip_status(launch_build_slices((const uint16_t*)cb, (uint16_t*)slices, hsq, dims->T / dims->Tc,
                                        dims->H_kv, dims->K * n_codebook_groups(dims), dims->c, dims->Tc,
                                        stream));
}

int loopvq_rope_table(int32_t max_pos, int32_t D, double base, float* table) {
  if (max_pos < 0 || (D != 64 && D != 128) || !(base > 1.0)) return LOOPVQ_ERR_INVALID_ARG;
  if (max_pos > 0 && table == nullptr) return LOOPVQ_ERR_INVALID_ARG;
  const int nch = D / 16;
  const int64_t padded = ((int64_t)max_pos + 15) / 16 * 16;
  for (int64_t p = 0; p < padded; ++p) {
    for (int j = 0; j < nch; ++j) {
      for (int i = 0; i < 4; ++i) {
        float* o = table + ((((size_t)(p >> 2) * nch + j) * 4 + i) * 4 + (p & 3)) * 4;
        for (int e = 0; e < 2; ++e) {
          const int f = i * (D / 8) + 2 * j + e;
          const double theta = pow(base, -2.0 * f / D);
          const double ang = (double)p * theta;
          o[2 * e] = (float)cos(ang);
          o[2 * e + 1] = (float)sin(ang);
        }
      }
    }
  }
  return LOOPVQ_OK;
}

size_t loopvq_rope_table_floats(int32_t max_pos, int32_t D) {
  if (max_pos < 0 || (D != 64 && D != 128)) return 0;
  return (size_t)(((int64_t)max_pos + 15) / 16 * 16) * D;
}

}  // extern "C"

// shared by the dense, paged-bf16 and TaSQ encode entry points: codes
// streams kv_lo .. kv_lo + kv_n - 1 of {K, V}, inputs fp32 when xf32
static int encode_impl(const loopvq_dims* dims, int32_t n_tok, int32_t first_block, int32_t n_blocks,
                       const void* xk, const void* xv, const int32_t* src_slot, int64_t step_stride,
                       const void* cb, const float* hsq, const int32_t* slot_mapping, uint8_t* index_cache,
                       int64_t block_stride_bytes, int kv_lo, int kv_n, bool xf32, int32_t* near_tie,
                       hipStream_t stream) {
  int st = check_dims(dims);
  if (st != LOOPVQ_OK) return st;
  const int nb_total = dims->T / dims->Tc;
  if (n_tok < 0 || first_block < 0 || n_blocks < 1 || first_block + n_blocks > nb_total)
    return LOOPVQ_ERR_INVALID_ARG;
  if (n_blocks > 1 && block_stride_bytes <= 0) return LOOPVQ_ERR_INVALID_ARG;
  // 4-bit rows pack the codes of groups g, g^1 into one byte: 16 groups or more
  if ((dims->D / dims->c) % (dims->bits == 4 ? 16 : 8) != 0) return LOOPVQ_ERR_UNSUPPORTED;
  if (n_tok == 0) return LOOPVQ_OK;
  if (!xk || !xv || !cb || !hsq || !slot_mapping || !index_cache) return LOOPVQ_ERR_INVALID_ARG;
  const int H = dims->H_kv, K = dims->K * n_codebook_groups(dims), G = dims->c * dims->Tc;
  EncodeParams p{};
  p.xk = xk;
  p.xv = xv;
  p.src_slot = src_slot;
  p.step_stride = step_stride;
  p.cb = (const uint16_t*)cb + (size_t)first_block * H * 2 * K * G;
  p.hsq = hsq + (size_t)first_block * H * 2 * K;
  p.slot_mapping = slot_mapping;
  p.cache = index_cache;
  p.block_stride = block_stride_bytes;
  p.n_tok = n_tok;
  p.H_kv = H;
  p.D = dims->D;
  p.c = dims->c;
  p.Tc = dims->Tc;
  p.K = dims->K;
  p.log2P = ilog2(dims->page_size);
  p.per_group = dims->per_group;
  p.kv_lo = kv_lo;
  p.kv_n = kv_n;
  p.near_tie = near_tie;
  // units of 32 (token, group) vectors (per group: 32 tokens of one group);
  // about 8192 waves over the whole call
  const long long streams = (long long)n_blocks * kv_n * H * n_codebook_groups(dims);
  const long long units = dims->per_group ? ((long long)n_tok + 31) / 32
                                          : ((long long)n_tok * (dims->D / dims->c) + 31) / 32;
  long long upw = (streams * units + 8191) / 8192;
  upw = std::max<long long>(1, std::min<long long>(upw, units));
  p.units_per_wave = (int)upw;
  p.n_unit_groups = (int)((units + 4 * upw - 1) / (4 * upw));
  // fp32 input needs the fp32 instantiation (G = 8 exists only there)
  if (!xf32 && G == 8) return LOOPVQ_ERR_UNSUPPORTED;
  return hip_status(launch_encode(G, xf32, dims->bits, p, n_blocks, stream));
}

extern "C" {

int loopvq_encode(const loopvq_dims* dims, int32_t n_tok, int32_t first_block, int32_t n_blocks,
                  const void* xk, const void* xv, const void* cb, const float* hsq,
                  const int32_t* slot_mapping, uint8_t* index_cache, int64_t block_stride_bytes,
                  int32_t* near_tie_count, hipStream_t stream) {
  if (check_dims(dims) != LOOPVQ_OK) return check_dims(dims);
  if (((uintptr_t)near_tie_count & 3) != 0) return LOOPVQ_ERR_INVALID_ARG;
  const int64_t step_stride = (int64_t)std::max(n_tok, 0) * dims->H_kv * dims->D;
  return encode_impl(dims, n_tok, first_block, n_blocks, xk, xv, nullptr, step_stride, cb, hsq, slot_mapping,
                     index_cache, block_stride_bytes, 0, 2, dims->x_dtype == LOOPVQ_DTYPE_F32, near_tie_count,
                     stream);
}

int loopvq_encode_pages(const loopvq_dims* dims, int32_t n_tok, int32_t first_block, int32_t n_blocks,
                        const void* kv_pages, int64_t step_stride, const int32_t* src_slot, const void* cb,
                        const float* hsq, const int32_t* slot_mapping, uint8_t* index_cache,
                        int64_t block_stride_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != LOOPVQ_OK) return st;
  if (dims->x_dtype != LOOPVQ_DTYPE_BF16) return LOOPVQ_ERR_UNSUPPORTED;   // the window pages are bf16
  if (n_tok > 0 && (!kv_pages || !src_slot)) return LOOPVQ_ERR_INVALID_ARG;
  if (n_tok > 0 && ((uintptr_t)kv_pages & 15) != 0) return LOOPVQ_ERR_INVALID_ARG;
  if (n_blocks * dims->Tc > 1 && step_stride <= 0) return LOOPVQ_ERR_INVALID_ARG;
  if (step_stride < 0 || step_stride % 8 != 0) return LOOPVQ_ERR_INVALID_ARG;
  // block beta of this call reads loop steps (beta - first_block)*Tc .. of the pools
  const void* xv = kv_pages ? (const void*)((const uint16_t*)kv_pages + 8 * dims->D) : nullptr;
  return encode_impl(dims, n_tok, first_block, n_blocks, kv_pages, xv, src_slot, step_stride, cb, hsq,
                     slot_mapping, index_cache, block_stride_bytes, 0, 2, false, nullptr, stream);
}

size_t loopvq_encode_tasq_workspace_bytes(const loopvq_dims* dims, int32_t n_tok, int32_t n_blocks) {
  if (check_dims(dims) != LOOPVQ_OK || n_tok < 0 || n_blocks < 0) return 0;
  return align256((size_t)n_blocks * dims->Tc * n_tok * dims->H_kv * dims->D * sizeof(float));
}

int loopvq_encode_tasq(const loopvq_dims* dims, int32_t n_tok, int32_t first_block, int32_t n_blocks,
                       const void* xk, const void* xv, const loopvq_tasq* tasq, const void* cb,
                       const float* hsq, const int32_t* slot_mapping, uint8_t* index_cache,
                       int64_t block_stride_bytes, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  int st = check_tasq(dims, tasq);
  if (st != LOOPVQ_OK) return st;
  const int nb_total = dims->T / dims->Tc;
  if (n_tok < 0 || first_block < 0 || n_blocks < 1 || first_block + n_blocks > nb_total)
    return LOOPVQ_ERR_INVALID_ARG;
  if (n_tok == 0) return LOOPVQ_OK;
  if (!xk || !xv || !slot_mapping || !workspace) return LOOPVQ_ERR_INVALID_ARG;
  if (((uintptr_t)workspace & 255) != 0) return LOOPVQ_ERR_INVALID_ARG;
  // the transform reads keys and weights in 16-byte runs
  if (((uintptr_t)xk & 15) != 0 || ((uintptr_t)tasq->w & 15) != 0) return LOOPVQ_ERR_INVALID_ARG;
  if (workspace_bytes < loopvq_encode_tasq_workspace_bytes(dims, n_tok, n_blocks)) return LOOPVQ_ERR_WORKSPACE;
  // the rest of the checks are the encoder's, made before anything is launched
  if (!cb || !hsq || !index_cache || (n_blocks > 1 && block_stride_bytes <= 0)) return LOOPVQ_ERR_INVALID_ARG;
  if ((dims->D / dims->c) % (dims->bits == 4 ? 16 : 8) != 0) return LOOPVQ_ERR_UNSUPPORTED;
  TasqParams tp{};
  tp.xk = xk;
  tp.w = tasq->w;
  tp.perm = tasq->perm;
  tp.slot_mapping = slot_mapping;
  tp.sigma = tasq->sigma;
  tp.sigma_stride = tasq->sigma_stride;
  tp.u = (float*)workspace;
  tp.n_tok = n_tok;
  tp.H = dims->H_kv;
  tp.D = dims->D;
  tp.Tc = dims->Tc;
  tp.first_step = first_block * dims->Tc;
  st = hip_status(launch_tasq_transform(dims->x_dtype == LOOPVQ_DTYPE_F32, tp, n_blocks * dims->Tc, stream));
  if (st != LOOPVQ_OK) return st;
  const int64_t step_stride = (int64_t)n_tok * dims->H_kv * dims->D;
  // keys: the codes of u (fp32); values: as loopvq_encode
  st = encode_impl(dims, n_tok, first_block, n_blocks, workspace, workspace, nullptr, step_stride, cb, hsq,
                   slot_mapping, index_cache, block_stride_bytes, 0, 1, true, nullptr, stream);
  if (st != LOOPVQ_OK) return st;
  return encode_impl(dims, n_tok, first_block, n_blocks, xv, xv, nullptr, step_stride, cb, hsq, slot_mapping,
                     index_cache, block_stride_bytes, 1, 1, dims->x_dtype == LOOPVQ_DTYPE_F32, nullptr, stream);
}

size_t loopvq_kmeans_workspace_bytes(const loopvq_dims* dims, int32_t n_blocks) {
  if (check_dims(dims) != LOOPVQ_OK || n_blocks < 0) return 0;
  const size_t per = (size_t)dims->K * dims->c * dims->Tc + dims->K + 2;
  return align256((size_t)n_blocks * 2 * dims->H_kv * per * sizeof(double));
}

int loopvq_kmeans_update(const loopvq_dims* dims, int32_t n_tok, int32_t first_block, int32_t n_blocks,
                         const void* xk, const void* xv, const int32_t* slot_mapping, const uint8_t* index_cache,
                         int64_t block_stride_bytes, const void* cb, void* cb_out, double* err, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != LOOPVQ_OK) return st;
  if (dims->per_group) return LOOPVQ_ERR_UNSUPPORTED;
  const int nb_total = dims->T / dims->Tc;
  if (n_tok < 0 || first_block < 0 || n_blocks < 1 || first_block + n_blocks > nb_total)
    return LOOPVQ_ERR_INVALID_ARG;
  if (n_blocks > 1 && block_stride_bytes <= 0) return LOOPVQ_ERR_INVALID_ARG;
  if (!cb || !cb_out || !workspace) return LOOPVQ_ERR_INVALID_ARG;
  if (n_tok > 0 && (!xk || !xv || !slot_mapping || !index_cache)) return LOOPVQ_ERR_INVALID_ARG;
  if (((uintptr_t)workspace & 255) != 0) return LOOPVQ_ERR_INVALID_ARG;
  if (workspace_bytes < loopvq_kmeans_workspace_bytes(dims, n_blocks)) return LOOPVQ_ERR_WORKSPACE;
  const int H = dims->H_kv, K = dims->K, G = dims->c * dims->Tc;
  KmeansParams p{};
  p.xk = xk;
  p.xv = xv;
  p.slot_mapping = slot_mapping;
  p.cache = index_cache;
  p.block_stride = block_stride_bytes;
  p.cb = (const uint16_t*)cb + (size_t)first_block * H * 2 * K * G;
  p.cb_out = (uint16_t*)cb_out + (size_t)first_block * H * 2 * K * G;
  p.err = err;
  p.gsum = (double*)workspace;
  p.n_tok = n_tok;
  p.H_kv = H;
  p.D = dims->D;
  p.c = dims->c;
  p.Tc = dims->Tc;
  p.K = K;
  p.bits = dims->bits;
  p.log2P = ilog2(dims->page_size);
  // about 2048 workgroups over the call
  const long long streams = (long long)n_blocks * 2 * H;
  p.tok_per_wg = (int)std::max<long long>(16, ((long long)n_tok * streams + 2047) / 2048);
  return hip_status(launch_kmeans_update(dims->x_dtype == LOOPVQ_DTYPE_F32, p, n_blocks, stream));
}

size_t loopvq_decode_workspace_bytes(const loopvq_dims* dims, int32_t B, int32_t max_seq_len) {
  if (check_dims(dims) != LOOPVQ_OK || B < 0 || max_seq_len < 0) return 0;
  const DecodePlan pl = plan_decode(dims, B, max_seq_len);
  return pl.total();
}

static int check_decode_common(const loopvq_dims* dims, int32_t B, int32_t max_seq_len) {
  int st = check_dims(dims);
  if (st != LOOPVQ_OK) return st;
  if (B < 0 || max_seq_len < 0) return LOOPVQ_ERR_INVALID_ARG;
  if (!decode_supported(dims->D, dims->c, dims->bits)) return LOOPVQ_ERR_UNSUPPORTED;
  return LOOPVQ_OK;
}

}  // extern "C"

// the split pass over the coded positions [seq_lo[b], seq_end[b]) of each
// request (seq_lo null: from 0)
static int split_impl(const loopvq_dims* dims, int32_t t, int32_t B, const void* q,
                      const uint8_t* index_cache, const void* slices, const float* rope_table,
                      int32_t max_pos, const int32_t* block_table, int32_t max_pages,
                      const int32_t* seq_lens, const int32_t* seq_lo, int32_t max_seq_len, float sm_scale,
                      void* workspace, size_t workspace_bytes, const loopvq_tasq* tasq, hipStream_t stream) {
  int st = check_decode_common(dims, B, max_seq_len);
  if (st != LOOPVQ_OK) return st;
  if (t < 1 || t > dims->T || max_pos < 0 || max_pages < 0) return LOOPVQ_ERR_INVALID_ARG;
  if (max_seq_len > max_pos || (long long)max_seq_len > (long long)max_pages * dims->page_size)
    return LOOPVQ_ERR_INVALID_ARG;
  if (B == 0) return LOOPVQ_OK;
  if (!q || !index_cache || !slices || !rope_table || !block_table || !seq_lens || !workspace)
    return LOOPVQ_ERR_INVALID_ARG;
  if (((uintptr_t)workspace & 255) != 0) return LOOPVQ_ERR_INVALID_ARG;
  const DecodePlan pl = plan_decode(dims, B, max_seq_len);
  if (workspace_bytes < pl.total()) return LOOPVQ_ERR_WORKSPACE;

  DecodeParams p{};
  p.q = q;
  p.cache = index_cache;
  p.slices = (const uint16_t*)slices + (size_t)(t - 1) * dims->H_kv * 2 * dims->K * n_codebook_groups(dims) * dims->c;
  p.rope = rope_table;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.seq_lo = seq_lo;
  p.part_o = (float*)workspace;
  p.part_lse = (float*)((char*)workspace + pl.bytes_o);
  p.B = B;
  p.H_kv = dims->H_kv;
  p.H_q = dims->H_q;
  p.grp = pl.grp;
  p.max_pages = max_pages;
  p.log2P = ilog2(dims->page_size);
  p.n_pairs = pl.n_pairs;
  p.n_dg = pl.n_dg;
  p.quad = pl.quad;
  p.shared_rope = pl.shared_rope;
  p.Lc = pl.Lc;
  p.n_chunks = pl.n_chunks;
  p.items_per_head = pl.items_per_head;
  p.wg_per_head = pl.wg_per_head;
  p.max_seq_len = max_seq_len;
  const float scale = sm_scale > 0.f ? sm_scale : 1.0f / sqrtf((float)dims->D);
  p.scale_log2 = scale * 1.4426950408889634f;
  const bool qf32 = dims->io_dtype == LOOPVQ_DTYPE_F32;
  int grid = pl.grid;
  if (tasq == nullptr && pl.quad && pl.shared_rope && B <= DECODE_SORT_MAX && pl.n_dg / 8 <= 64) {
    // quads in order of decreasing work: about one workgroup per CU, each
    // keeping its head's slices in LDS and walking the items of its ranks (a
    // larger grid would only add workgroups that find no item)
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && ncu > 0)
      grid = dims->H_kv * std::min(pl.wg_per_head, std::max(1, ncu / dims->H_kv));
  }
  if (tasq != nullptr && pl.quad) {
    // the TaSQ kernel serves duos: the plan's chunks (and so the workspace)
    // stay, with two waves per quad's pairs
    p.quad = 0;
    p.n_dg = std::max(1, (pl.n_pairs + 1) / 2);
    p.items_per_head = p.n_dg * pl.n_chunks;
    p.wg_per_head = (p.items_per_head + 7) / 8;
    grid = dims->H_kv * p.wg_per_head;
  }
  if (tasq != nullptr) {
    // step t's weights, its block's permutations and its sigma array
    p.tq_w = tasq->w + (size_t)(t - 1) * dims->H_kv * dims->D;
    p.tq_perm = tasq->perm + (size_t)((t - 1) / dims->Tc) * dims->H_kv * (dims->D / 2);
    p.tq_sigma = tasq->sigma + (size_t)(t - 1) * tasq->sigma_stride;
    return hip_status(launch_decode_split_tq(dims->D, dims->c, dims->bits, qf32, p, grid, stream));
  }
  if (dims->per_group) return hip_status(launch_decode_split_pg(dims->D, dims->c, dims->bits, qf32, p, grid, stream));
  return hip_status(launch_decode_split(dims->D, dims->c, dims->bits, qf32, p, grid, stream));
}

// the combine pass; win_o / win_lse: the bf16-token partials, or null
static int combine_impl(const loopvq_dims* dims, int32_t B, const int32_t* seq_lens, int32_t max_seq_len,
                        void* out, float* lse, const void* workspace, size_t workspace_bytes,
                        bool with_window, hipStream_t stream) {
  int st = check_decode_common(dims, B, max_seq_len);
  if (st != LOOPVQ_OK) return st;
  if (B == 0) return LOOPVQ_OK;
  if (!seq_lens || !out || !workspace) return LOOPVQ_ERR_INVALID_ARG;
  if (((uintptr_t)workspace & 255) != 0) return LOOPVQ_ERR_INVALID_ARG;
  const DecodePlan pl = plan_decode(dims, B, max_seq_len);
  if (workspace_bytes < pl.total()) return LOOPVQ_ERR_WORKSPACE;
  CombineParams cp{};
  cp.part_o = (const float*)workspace;
  cp.part_lse = (const float*)((const char*)workspace + pl.bytes_o);
  if (with_window) {
    cp.win_o = (const float*)((const char*)workspace + pl.bytes_o + pl.bytes_lse);
    cp.win_lse = (const float*)((const char*)workspace + pl.bytes_o + pl.bytes_lse + pl.bytes_wo);
  }
  cp.seq_lens = seq_lens;
  cp.out = out;
  cp.lse = lse;
  cp.B = B;
  cp.H_q = dims->H_q;
  cp.grp = pl.grp;
  cp.n_pairs = pl.n_pairs;
  cp.n_chunks = pl.n_chunks;
  cp.Lc = pl.Lc;
  cp.max_seq_len = max_seq_len;
  return hip_status(launch_decode_combine(dims->D, dims->io_dtype == LOOPVQ_DTYPE_BF16, cp, stream));
}

extern "C" {

int loopvq_decode_split(const loopvq_dims* dims, int32_t t, int32_t B, const void* q,
                        const uint8_t* index_cache, const void* slices, const float* rope_table,
                        int32_t max_pos, const int32_t* block_table, int32_t max_pages,
                        const int32_t* seq_lens, int32_t max_seq_len, float sm_scale, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  return split_impl(dims, t, B, q, index_cache, slices, rope_table, max_pos, block_table, max_pages, seq_lens,
                    nullptr, max_seq_len, sm_scale, workspace, workspace_bytes, nullptr, stream);
}

int loopvq_decode_combine(const loopvq_dims* dims, int32_t B, const int32_t* seq_lens, int32_t max_seq_len,
                          void* out, float* lse, const void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  return combine_impl(dims, B, seq_lens, max_seq_len, out, lse, workspace, workspace_bytes, false, stream);
}

int loopvq_decode_attn(const loopvq_dims* dims, int32_t t, int32_t B, const void* q,
                       const uint8_t* index_cache, const void* slices, const float* rope_table,
                       int32_t max_pos, const int32_t* block_table, int32_t max_pages,
                       const int32_t* seq_lens, int32_t max_seq_len, float sm_scale, void* out,
                       float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_decode_common(dims, B, max_seq_len);
  if (st != LOOPVQ_OK) return st;
  if (B > 0 && out == nullptr) return LOOPVQ_ERR_INVALID_ARG;
  st = loopvq_decode_split(dims, t, B, q, index_cache, slices, rope_table, max_pos, block_table, max_pages,
                           seq_lens, max_seq_len, sm_scale, workspace, workspace_bytes, stream);
  if (st != LOOPVQ_OK) return st;
  return loopvq_decode_combine(dims, B, seq_lens, max_seq_len, out, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"

// coded positions through the split pass, bf16 sink and window through the
// window kernel, then the combine; tasq: TaSQ-coded keys, or null
static int window_impl(const loopvq_dims* dims, int32_t t, int32_t B, const void* q,
                       const uint8_t* index_cache, const void* slices, const float* rope_table,
                       int32_t max_pos, const int32_t* block_table, int32_t max_pages,
                       const int32_t* seq_lens, int32_t max_seq_len, const loopvq_bf16_window* window,
                       float sm_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                       const loopvq_tasq* tasq, hipStream_t stream) {
  int st = check_decode_common(dims, B, max_seq_len);
  if (st != LOOPVQ_OK) return st;
  if (window == nullptr) return LOOPVQ_ERR_INVALID_ARG;
  if (t < 1 || t > dims->T || max_pos < 0 || max_pages < 0 || window->max_pages < 1) return LOOPVQ_ERR_INVALID_ARG;
  if (max_seq_len > max_pos || (long long)max_seq_len > (long long)max_pages * dims->page_size)
    return LOOPVQ_ERR_INVALID_ARG;
  if (B == 0) return LOOPVQ_OK;
  if (!q || !index_cache || !slices || !rope_table || !block_table || !seq_lens || !out || !workspace)
    return LOOPVQ_ERR_INVALID_ARG;
  if (!window->kv || !window->page_table || !window->n_sink || !window->win_start) return LOOPVQ_ERR_INVALID_ARG;
  if (((uintptr_t)window->kv & 15) != 0 || ((uintptr_t)workspace & 255) != 0) return LOOPVQ_ERR_INVALID_ARG;
  const DecodePlan pl = plan_decode(dims, B, max_seq_len);
  if (workspace_bytes < pl.total()) return LOOPVQ_ERR_WORKSPACE;
  // coded positions [n_sink, win_start)
  st = split_impl(dims, t, B, q, index_cache, slices, rope_table, max_pos, block_table, max_pages,
                  window->win_start, window->n_sink, max_seq_len, sm_scale, workspace, workspace_bytes, tasq,
                  stream);
  if (st != LOOPVQ_OK) return st;
  WindowParams wp{};
  wp.q = q;
  wp.kv = (const uint16_t*)window->kv;
  wp.page_table = window->page_table;
  wp.n_sink = window->n_sink;
  wp.win_start = window->win_start;
  wp.seq_lens = seq_lens;
  wp.rope = rope_table;
  wp.win_o = (float*)((char*)workspace + pl.bytes_o + pl.bytes_lse);
  wp.win_lse = (float*)((char*)workspace + pl.bytes_o + pl.bytes_lse + pl.bytes_wo);
  wp.H_kv = dims->H_kv;
  wp.H_q = dims->H_q;
  wp.grp = pl.grp;
  wp.n_pairs = pl.n_pairs;
  wp.max_pages = window->max_pages;
  wp.max_seq_len = max_seq_len;
  const float scale = sm_scale > 0.f ? sm_scale : 1.0f / sqrtf((float)dims->D);
  wp.scale_log2 = scale * 1.4426950408889634f;
  st = hip_status(launch_decode_window(dims->D, dims->io_dtype == LOOPVQ_DTYPE_F32, wp, B, stream));
  if (st != LOOPVQ_OK) return st;
  return combine_impl(dims, B, window->win_start, max_seq_len, out, lse, workspace, workspace_bytes, true, stream);
}

extern "C" {

int loopvq_decode_attn_window(const loopvq_dims* dims, int32_t t, int32_t B, const void* q,
                              const uint8_t* index_cache, const void* slices, const float* rope_table,
                              int32_t max_pos, const int32_t* block_table, int32_t max_pages,
                              const int32_t* seq_lens, int32_t max_seq_len, const loopvq_bf16_window* window,
                              float sm_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  return window_impl(dims, t, B, q, index_cache, slices, rope_table, max_pos, block_table, max_pages, seq_lens,
                     max_seq_len, window, sm_scale, out, lse, workspace, workspace_bytes, nullptr, stream);
}

int loopvq_decode_attn_tasq(const loopvq_dims* dims, int32_t t, int32_t B, const void* q,
                            const uint8_t* index_cache, const void* slices, const float* rope_table,
                            int32_t max_pos, const int32_t* block_table, int32_t max_pages,
                            const int32_t* seq_lens, int32_t max_seq_len, const loopvq_tasq* tasq,
                            const loopvq_bf16_window* window, float sm_scale, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_decode_common(dims, B, max_seq_len);
  if (st != LOOPVQ_OK) return st;
  st = check_tasq(dims, tasq);
  if (st != LOOPVQ_OK) return st;
  if (window != nullptr)
    return window_impl(dims, t, B, q, index_cache, slices, rope_table, max_pos, block_table, max_pages, seq_lens,
                       max_seq_len, window, sm_scale, out, lse, workspace, workspace_bytes, tasq, stream);
  if (B > 0 && out == nullptr) return LOOPVQ_ERR_INVALID_ARG;
  st = split_impl(dims, t, B, q, index_cache, slices, rope_table, max_pos, block_table, max_pages, seq_lens,
                  nullptr, max_seq_len, sm_scale, workspace, workspace_bytes, tasq, stream);
  if (st != LOOPVQ_OK) return st;
  return combine_impl(dims, B, seq_lens, max_seq_len, out, lse, workspace, workspace_bytes, false, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- no-allocation decode
// The split partials of loopvq_decode_attn_noalloc live in this fixed array.
// Each GPU holds its own copy at its own address; host code never uses the
// name itself as an address (on the host it is only a stand-in for the
// symbol), only the device address looked up for the current device.
static __device__ __align__(256) uint8_t scratch[LOOPVQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[SCRATCH_MAX_DEVICES];   // device address of scratch, per device id

// address of the current device's copy, looked up once per device
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return LOOPVQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return LOOPVQ_ERR_HIP;
    scratch_dev[dev] = ptr;
  }
  *out = scratch_dev[dev];
  return LOOPVQ_OK;
}

}  // namespace

extern "C" {

int loopvq_decode_attn_noalloc(const loopvq_dims* dims, int32_t t, int32_t B, const void* q,
                               const uint8_t* index_cache, const void* slices, const float* rope_table,
                               int32_t max_pos, const int32_t* block_table, int32_t max_pages,
                               const int32_t* seq_lens, int32_t max_seq_len, float sm_scale, void* out,
                               float* lse, hipStream_t stream) {
  int st = check_decode_common(dims, B, max_seq_len);
  if (st != LOOPVQ_OK) return st;
  if (plan_decode(dims, B, max_seq_len).total() > (size_t)LOOPVQ_NOALLOC_SCRATCH_BYTES) return LOOPVQ_ERR_SCRATCH;
  void* ws = nullptr;
  if (B > 0) {
    st = scratch_on_current_device(&ws);
    if (st != LOOPVQ_OK) return st;
  }
  return loopvq_decode_attn(dims, t, B, q, index_cache, slices, rope_table, max_pos, block_table, max_pages,
                            seq_lens, max_seq_len, sm_scale, out, lse, ws,
                            ws != nullptr ? (size_t)LOOPVQ_NOALLOC_SCRATCH_BYTES : 0, stream);
}

}  // extern "C"
