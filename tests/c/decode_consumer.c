/*
 * A plain C11 program that runs LoopVQ decode attention through
 * include/loopvq.h with the HIP runtime only (no PyTorch in the process):
 * it builds the codebook slices and the RoPE table, copies the inputs to the
 * device, calls loopvq_decode_attn and writes the output back.
 *
 * usage: decode_consumer DIR
 *   DIR/meta.txt   D c Tc T bits H_kv H_q page_size B t max_seq_len max_pages num_pages
 *   DIR/cb.bin     fp16 codebooks [T/Tc][H_kv][2][K][c*Tc]
 *   DIR/q.bin      bf16 queries [B][H_q][D]
 *   DIR/cache.bin  index cache of block (t-1)/Tc: [num_pages][H_kv][2][P][R] bytes
 *   DIR/bt.bin     int32 block table [B][max_pages]
 *   DIR/lens.bin   int32 seq_lens [B]
 * writes DIR/out.bin (bf16 [B][H_q][D]) and DIR/lse.bin (fp32 [B][H_q]).
 * Exit status 0 on success; a failed call prints its status string.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "loopvq.h"

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (f == NULL) return NULL;
  void* buf = malloc(bytes > 0 ? bytes : 1);
  const size_t got = buf != NULL ? fread(buf, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(buf);
    return NULL;
  }
  return buf;
}

static int write_file(const char* dir, const char* name, const void* data, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (f == NULL) return -1;
  const size_t put = fwrite(data, 1, bytes, f);
  fclose(f);
  return put == bytes ? 0 : -1;
}

#define HIP_OK(call)                                                           \
  do {                                                                         \
    hipError_t e_ = (call);                                                    \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));       \
      return 1;                                                                \
    }                                                                          \
  } while (0)

#define LVQ_OK(call)                                                           \
  do {                                                                         \
    int s_ = (call);                                                           \
    if (s_ != LOOPVQ_OK) {                                                     \
      fprintf(stderr, "%s failed: %s\n", #call, loopvq_status_string(s_));    \
      return 1;                                                                \
    }                                                                          \
  } while (0)

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes > 0 ? bytes : 1) != hipSuccess) return NULL;
  if (hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  char path[4096];
  snprintf(path, sizeof path, "%s/meta.txt", dir);
  FILE* mf = fopen(path, "r");
  if (mf == NULL) return 2;
  int D, c, Tc, T, bits, H_kv, H_q, P, B, t, max_seq_len, max_pages, num_pages;
  const int nread = fscanf(mf, "%d %d %d %d %d %d %d %d %d %d %d %d %d", &D, &c, &Tc, &T, &bits, &H_kv, &H_q, &P,
                           &B, &t, &max_seq_len, &max_pages, &num_pages);
  fclose(mf);
  if (nread != 13) return 2;

  loopvq_dims d;
  memset(&d, 0, sizeof d);
  d.D = D;
  d.c = c;
  d.Tc = Tc;
  d.T = T;
  d.bits = bits;
  d.K = 1 << bits;
  d.H_kv = H_kv;
  d.H_q = H_q;
  d.page_size = P;
  d.x_dtype = LOOPVQ_DTYPE_BF16;
  d.io_dtype = LOOPVQ_DTYPE_BF16;
  const int R = loopvq_row_bytes(&d);
  if (R <= 0) return 2;

  const size_t G = (size_t)c * Tc, K = (size_t)d.K;
  const size_t cb_bytes = (size_t)(T / Tc) * H_kv * 2 * K * G * 2;
  const size_t sl_bytes = (size_t)T * H_kv * 2 * K * c * 2;
  const size_t q_bytes = (size_t)B * H_q * D * 2;
  const size_t cache_bytes = (size_t)num_pages * H_kv * 2 * P * R;
  const size_t bt_bytes = (size_t)B * max_pages * 4;
  const size_t lens_bytes = (size_t)B * 4;
  void* cb = read_file(dir, "cb.bin", cb_bytes);
  void* q = read_file(dir, "q.bin", q_bytes);
  void* cache = read_file(dir, "cache.bin", cache_bytes);
  void* bt = read_file(dir, "bt.bin", bt_bytes);
  void* lens = read_file(dir, "lens.bin", lens_bytes);
  if (!cb || !q || !cache || !bt || !lens) {
    fprintf(stderr, "missing or short input file\n");
    return 2;
  }

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  void* cb_d = to_device(cb, cb_bytes);
  void* q_d = to_device(q, q_bytes);
  void* cache_d = to_device(cache, cache_bytes);
  void* bt_d = to_device(bt, bt_bytes);
  void* lens_d = to_device(lens, lens_bytes);
  if (!cb_d || !q_d || !cache_d || !bt_d || !lens_d) {
    fprintf(stderr, "device allocation or copy failed\n");
    return 1;
  }

  /* slices once per layer, the RoPE table once per process */
  void* slices_d = NULL;
  HIP_OK(hipMalloc(&slices_d, sl_bytes));
  LVQ_OK(loopvq_build_codebook_slices(&d, cb_d, slices_d, NULL, stream));
  const size_t nrope = loopvq_rope_table_floats(max_seq_len, D);
  float* rope = (float*)malloc(nrope * sizeof(float));
  if (rope == NULL) return 1;
  LVQ_OK(loopvq_rope_table(max_seq_len, D, 10000.0, rope));
  void* rope_d = to_device(rope, nrope * sizeof(float));
  if (rope_d == NULL) return 1;

  /* one decode call, then the outputs back to the host */
  const size_t ws_bytes = loopvq_decode_workspace_bytes(&d, B, max_seq_len);
  void *ws_d = NULL, *out_d = NULL, *lse_d = NULL;
  HIP_OK(hipMalloc(&ws_d, ws_bytes));
  HIP_OK(hipMalloc(&out_d, q_bytes));
  HIP_OK(hipMalloc(&lse_d, (size_t)B * H_q * 4));
  LVQ_OK(loopvq_decode_attn(&d, t, B, q_d, (const uint8_t*)cache_d, slices_d, (const float*)rope_d, max_seq_len,
                            (const int32_t*)bt_d, max_pages, (const int32_t*)lens_d, max_seq_len, 0.0f, out_d,
                            (float*)lse_d, ws_d, ws_bytes, stream));
  HIP_OK(hipStreamSynchronize(stream));
  void* out = malloc(q_bytes);
  void* lse = malloc((size_t)B * H_q * 4);
  if (out == NULL || lse == NULL) return 1;
  HIP_OK(hipMemcpy(out, out_d, q_bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse, lse_d, (size_t)B * H_q * 4, hipMemcpyDeviceToHost));
  if (write_file(dir, "out.bin", out, q_bytes) != 0 || write_file(dir, "lse.bin", lse, (size_t)B * H_q * 4) != 0)
    return 1;

  hipFree(cb_d);
  hipFree(q_d);
  hipFree(cache_d);
  hipFree(bt_d);
  hipFree(lens_d);
  hipFree(slices_d);
  hipFree(rope_d);
  hipFree(ws_d);
  hipFree(out_d);
  hipFree(lse_d);
  HIP_OK(hipStreamDestroy(stream));
  free(cb);
  free(q);
  free(cache);
  free(bt);
  free(lens);
  free(rope);
  free(out);
  free(lse);
  printf("ok\n");
  return 0;
}
