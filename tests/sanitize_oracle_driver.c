/* Calls every entry point of the CPU oracle (oracle/gqref.c) on small
 * seeded inputs with ragged lengths, for a build under AddressSanitizer,
 * LeakSanitizer and UBSan (tests/test_sanitizers.py).  Exit status 0 when
 * every call returns success; the sanitizers abort on any memory error,
 * leak or undefined behaviour.  The results are not checked here: the
 * oracle's pins check them. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/gqref.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static float next_value(void) {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  const int64_t v = (int64_t)(rng >> 40) - (1 << 23);
  return (float)v * 1e-9f;
}

static int64_t code_bytes(int bits, int dense_w, int64_t n) {
  if (dense_w > 0) return (((n + 7) / 8) * dense_w + 7) / 8;
  return (n * bits + 7) / 8;
}

static int fail(const char *what) {
  fprintf(stderr, "oracle call failed: %s\n", what);
  return 1;
}

static int one_scheme(int scheme, int d, int s, int L, int flags, int64_t n) {
  const int bits = gqref_bits(scheme, s, L);
  const int k = gqref_meta_per_bucket(scheme, L);
  const int A = scheme == 0 ? 2 * s + 1 : (scheme == 3 ? L : 2);
  const int dense_w = (flags & 2) ? gqref_dense_width(A) : 0;
  const int64_t nb = (n + d - 1) / d, cb = code_bytes(bits, dense_w, n);
  float *g = malloc(n * sizeof(float)), *e = malloc(n * sizeof(float));
  float *x = malloc(n * sizeof(float)), *out = malloc(n * sizeof(float));
  float *meta = malloc(nb * k * sizeof(float));
  uint8_t *codes = malloc(cb > 0 ? cb : 1), *tie = malloc(nb);
  for (int64_t i = 0; i < n; ++i) {
    g[i] = next_value();
    e[i] = 0.01f * next_value();
  }
  int rc = 0;
  if (gqref_quantize(scheme, d, s, L, flags, 3.0f, (int64_t)d << 12, n, g, e, 5, 1, codes, meta, tie))
    rc = fail("quantize");
  if (!rc && gqref_select_levels(scheme, d, s, L, flags, 3.0f, (int64_t)d << 12, n, g, e, meta, tie))
    rc = fail("select_levels");
  if (!rc && gqref_quantize(scheme, d, s, L, flags, 3.0f, 0, n, g, NULL, 5, 0, codes, meta, tie))
    rc = fail("quantize without error feedback");
  if (!rc && gqref_dequantize(scheme, d, s, L, flags, n, codes, meta, x))
    rc = fail("dequantize");
  if (!rc && gqref_error_feedback(scheme, d, s, L, flags, n, g, e, codes, meta))
    rc = fail("error_feedback");
  const uint8_t *cl[3] = {codes, codes, codes};
  const float *ml[3] = {meta, meta, meta};
  memcpy(out, x, n * sizeof(float));
  if (!rc && gqref_dequantize_accumulate(scheme, d, s, L, flags, n, 3, cl, ml,
                                         0.5f, 0.25f, out))
    rc = fail("dequantize_accumulate");
  free(g); free(e); free(x); free(out); free(meta); free(codes); free(tie);
  return rc;
}

int main(void) {
  int rc = 0;
  const int64_t ns[] = {1, 63, 1000, 4099};
  for (int t = 0; t < 4 && !rc; ++t) {
    const int64_t n = ns[t];
    rc |= one_scheme(0, 64, 1, 5, 0, n);
    rc |= one_scheme(0, 512, 4, 5, 2, n);
    rc |= one_scheme(0, 128, 127, 5, 4, n);
    rc |= one_scheme(1, 256, 4, 5, 0, n);
    rc |= one_scheme(2, 64, 4, 5, 0, n);
    rc |= one_scheme(2, 2048, 4, 5, 0, n);
    rc |= one_scheme(3, 512, 4, 9, 1, n);
    rc |= one_scheme(3, 512, 4, 5, 8, n);
    rc |= one_scheme(3, 512, 4, 3, 2 | 4, n);
    rc |= one_scheme(3, 64, 4, 2, 0, n);
  }
  /* per-layer scale, Top-K, Elias, packing, Philox */
  const int64_t n = 3000;
  const int64_t off[5] = {0, 0, 1, 1700, n};
  float *g = malloc(n * sizeof(float)), *e = calloc(n, sizeof(float));
  float *out = calloc(n, sizeof(float)), *meta = malloc(4 * 64 * sizeof(float));
  uint8_t *codes = malloc(n);
  for (int64_t i = 0; i < n; ++i) g[i] = next_value();
  if (!rc && gqref_quantize_layers(4, 0, n, 4, off, g, e, 3, 0, codes, meta))
    rc = fail("quantize_layers");
  const uint8_t *cl[2] = {codes, codes};
  const float *ml[2] = {meta, meta};
  if (!rc && gqref_dequantize_accumulate_layers(4, 0, n, 4, off, 2, cl, ml, 0.5f, 0.f, out))
    rc = fail("dequantize_accumulate_layers");
  const int words = gqref_topk_record_words(64, 4, 5);
  const int64_t nbt = (n + 63) / 64;
  uint8_t *rec = malloc(nbt * words * 4);
  if (!rc && gqref_quantize_topk(64, 4, 5, 0, n, g, e, 3, 0, rec, meta))
    rc = fail("quantize_topk");
  const uint8_t *rl[1] = {rec};
  const float *tl[1] = {meta};
  if (!rc && gqref_dequantize_accumulate_topk(64, 4, 5, 0, n, 1, rl, tl, 1.f, 0.f, out))
    rc = fail("dequantize_accumulate_topk");
  /* Elias: 4-bit codes of s = 4 from the uniform quantizer */
  uint8_t *c4 = malloc((n * 4 + 7) / 8), *back = malloc((n * 4 + 7) / 8);
  float *m4 = malloc(((n + 511) / 512) * sizeof(float));
  uint8_t *t4 = malloc((n + 511) / 512);
  if (!rc && gqref_quantize(0, 512, 4, 5, 0, 3.f, 0, n, g, NULL, 1, 0, c4, m4, t4))
    rc = fail("quantize for elias");
  const int64_t mw = gqref_elias_max_words(512, 4, n);
  uint64_t *eoff = malloc(((n + 511) / 512 + 1) * sizeof(uint64_t));
  uint32_t *words32 = malloc(mw * sizeof(uint32_t));
  if (!rc && gqref_elias_encode(512, 4, n, c4, eoff, words32)) rc = fail("elias_encode");
  if (!rc && gqref_elias_decode(512, 4, n, eoff, words32, back)) rc = fail("elias_decode");
  uint32_t *digits = malloc(n * sizeof(uint32_t)), *d2 = malloc(n * sizeof(uint32_t));
  for (int64_t i = 0; i < n; ++i) digits[i] = (uint32_t)(i % 9);
  uint8_t *dz = malloc(((n + 7) / 8) * gqref_dense_width(9) / 8 + 1);
  gqref_pack_dense(9, n, digits, dz);
  gqref_unpack_dense(9, n, dz, d2);
  uint8_t *pk = malloc((n * 3 + 7) / 8);
  for (int64_t i = 0; i < n; ++i) digits[i] &= 7;
  gqref_pack(3, n, digits, pk);
  gqref_unpack(3, n, pk, d2);
  uint32_t w4[4];
  gqref_philox(1, 2, 3, w4);
  uint32_t *blk = malloc(16 * 4 * sizeof(uint32_t));
  gqref_philox_blocks(7, (uint64_t)1 << 33, 16, 2, blk);
  free(g); free(e); free(out); free(meta); free(codes); free(rec); free(c4);
  free(back); free(m4); free(t4); free(eoff); free(words32); free(digits);
  free(d2); free(dz); free(pk); free(blk);
  if (rc == 0) printf("oracle driver: every entry point ran\n");
  return rc;
}
