/*
 * A plain C11 consumer of include/loopvq.h, built with gcc against
 * libloopvq.so by tests/test_c_consumer.py.  It uses only the host-side
 * parts of the interface (status strings, row sizes, the RoPE table,
 * workspace sizes and argument validation), so it runs without a GPU: every
 * call below either computes on the host or must fail its checks before
 * anything is launched.  Prints "ok" and returns 0, or names the first
 * failed check and returns 1.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "loopvq.h"

static int failures = 0;

#define CHECK(cond)                                                       \
  do {                                                                    \
    if (!(cond)) {                                                        \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

static loopvq_dims layer_dims(void) {
  /* one layer of the 1.4B looped model: D = 128, c = 4, Tc = T = 4, 8-bit */
  loopvq_dims d;
  memset(&d, 0, sizeof d);
  d.D = 128;
  d.c = 4;
  d.Tc = 4;
  d.T = 4;
  d.bits = 8;
  d.K = 256;
  d.H_kv = 16;
  d.H_q = 16;
  d.page_size = 64;
  d.x_dtype = LOOPVQ_DTYPE_BF16;
  d.io_dtype = LOOPVQ_DTYPE_BF16;
  d.per_group = 0;
  return d;
}

int main(void) {
  loopvq_dims d = layer_dims();

  /* status strings exist for every status and for unknown values */
  const int codes[] = {LOOPVQ_OK, LOOPVQ_ERR_INVALID_ARG, LOOPVQ_ERR_UNSUPPORTED, LOOPVQ_ERR_WORKSPACE,
                       LOOPVQ_ERR_HIP, LOOPVQ_ERR_SCRATCH, 12345};
  for (size_t i = 0; i < sizeof codes / sizeof codes[0]; ++i) {
    const char* s = loopvq_status_string(codes[i]);
    CHECK(s != NULL && s[0] != '\0');
  }

  /* index row: D/c codes of `bits` bits */
  CHECK(loopvq_row_bytes(&d) == 32);
  loopvq_dims d4 = d;
  d4.bits = 4;
  d4.K = 16;
  CHECK(loopvq_row_bytes(&d4) == 16);
  loopvq_dims bad = d;
  bad.K = 255; /* K must equal 1 << bits */
  CHECK(loopvq_row_bytes(&bad) < 0);
  CHECK(loopvq_row_bytes(NULL) < 0);

  /* RoPE table: padded to a multiple of 16 positions, D floats each; spot
     values against cos/sin of p * base^(-2f/D) at the documented offsets */
  const int max_pos = 37, D = 128;
  const size_t n = loopvq_rope_table_floats(max_pos, D);
  CHECK(n == (size_t)48 * D);
  float* tab = (float*)malloc(n * sizeof(float));
  CHECK(tab != NULL);
  if (tab != NULL) {
    CHECK(loopvq_rope_table(max_pos, D, 10000.0, tab) == LOOPVQ_OK);
    const int ps[] = {0, 1, 5, 36};
    double worst = 0.0;
    for (size_t k = 0; k < sizeof ps / sizeof ps[0]; ++k) {
      const int p = ps[k], g = p / 4, nn = p % 4;
      for (int j = 0; j < D / 16; ++j)
        for (int i = 0; i < 4; ++i) {
          const float* v = tab + (((size_t)(g * (D / 16) + j) * 4 + i) * 4 + nn) * 4;
          const int f = i * (D / 8) + 2 * j;
          const double t0 = p * pow(10000.0, -2.0 * f / D), t1 = p * pow(10000.0, -2.0 * (f + 1) / D);
          const double e[4] = {cos(t0), sin(t0), cos(t1), sin(t1)};
          for (int u = 0; u < 4; ++u) {
            const double err = fabs((double)v[u] - e[u]);
            if (err > worst) worst = err;
          }
        }
    }
    CHECK(worst <= 6e-8); /* one fp32 rounding of values in [-1, 1] */
    free(tab);
  }
  CHECK(loopvq_rope_table(-1, D, 10000.0, NULL) != LOOPVQ_OK);
  CHECK(loopvq_rope_table_floats(10, 100) == 0); /* D must be a multiple of 16 */

  /* decode workspace: grows with the context, zero on invalid arguments */
  const size_t w1 = loopvq_decode_workspace_bytes(&d, 16, 4096);
  const size_t w2 = loopvq_decode_workspace_bytes(&d, 16, 32768);
  CHECK(w1 > 0 && w2 >= w1);
  CHECK(loopvq_decode_workspace_bytes(&d, -1, 10) == 0);
  CHECK(loopvq_decode_workspace_bytes(&bad, 16, 4096) == 0);

  /* argument validation happens before any launch: null device pointers,
     a bad loop step or a short workspace come back as errors */
  int32_t dummy = 0;
  CHECK(loopvq_decode_attn(&d, 1, 2, NULL, NULL, NULL, NULL, 64, NULL, 1, NULL, 64, 0.0f, NULL, NULL, NULL, 0,
                           NULL) == LOOPVQ_ERR_INVALID_ARG);
  CHECK(loopvq_decode_attn(&d, 0, 2, &dummy, (const uint8_t*)&dummy, &dummy, (const float*)&dummy, 64,
                           &dummy, 1, &dummy, 64, 0.0f, &dummy, NULL, &dummy, 1 << 20, NULL) ==
        LOOPVQ_ERR_INVALID_ARG); /* t is 1-based */
  CHECK(loopvq_decode_attn(&bad, 1, 2, &dummy, (const uint8_t*)&dummy, &dummy, (const float*)&dummy, 64,
                           &dummy, 1, &dummy, 64, 0.0f, &dummy, NULL, &dummy, 1 << 20, NULL) < 0);
  CHECK(loopvq_encode(&d, 4, 0, 1, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL) ==
        LOOPVQ_ERR_INVALID_ARG);
  /* an empty batch is valid and does nothing */
  CHECK(loopvq_decode_attn(&d, 1, 0, NULL, NULL, NULL, NULL, 0, NULL, 0, NULL, 0, 0.0f, NULL, NULL, NULL, 0,
                           NULL) == LOOPVQ_OK);

  if (failures != 0) return 1;
  printf("ok\n");
  return 0;
}
