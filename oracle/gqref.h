/*
 * gqref — plain, slow CPU oracle for bucketed stochastic gradient
 * quantization with error feedback.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant table with the HIP library; it is written from the
 * method's description on the pages:
 *   - "gradient quantization for communication" (glossary), §How Gradient
 *     Quantization Works (quantize / dequantize / aggregate) and §Quantization
 *     Schemes (uniform, stochastic, error feedback);
 *   - "Optimal Gradient Quantization Condition for Communication-Efficient
 *     Distributed Training" (paper review), §Proposed method (BinGrad-b, ORQ
 *     greedy levels, clipping, buckets of d elements);
 *   - "Gradient Quantization" (glossary), the core-mechanism paragraph
 *     (max-abs scaling, INT8), the Stochastic Quantization bullet, the QSGD,
 *     error-feedback and ternary/binary paragraphs.
 *
 * Every routine works on elements [i0, i0 + n) of a flat fp32 gradient, where
 * i0 is the global index of the first element (a multiple of the bucket size
 * d).  i0 only enters the random-number counter; buckets are formed from i0,
 * the packed bitstream starts at bit 0 of codes[0], and meta row 0 belongs to
 * the bucket that starts at i0.
 *
 * Scheme numbers: 0 uniform (QSGD / ternary / INT8), 1 two-level sign split,
 * 2 two-level optimal split (BinGrad-b), 3 ORQ.  flags bit 0 = clip, bit 1 =
 * dense packing (digits: c + s for the uniform scheme, the code otherwise),
 * bit 2 = deterministic rounding to the nearest level (uniform and ORQ),
 * bit 3 = ORQ levels by recursive bisection instead of one at a time.
 *
 * Return value: 0 on success, -1 on an invalid argument.
 */
#ifndef GQREF_H
#define GQREF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Philox4x32-10 block for (key = seed, counter = (ctr lo, ctr hi, step, 0)). */
void gqref_philox(uint64_t seed, uint64_t ctr, uint32_t step, uint32_t out[4]);

/* nblocks consecutive counters ctr0, ctr0+1, ...: out[4*b .. 4*b+3]. */
void gqref_philox_blocks(uint64_t seed, uint64_t ctr0, int64_t nblocks,
                         uint32_t step, uint32_t *out);

/* bits per code and metadata floats per bucket for a scheme, or -1. */
int gqref_bits(int scheme, int s, int L);
int gqref_meta_per_bucket(int scheme, int L);

/* Quantize: p = g (+ e), per-bucket levels, random rounding, packing;
 * with e != NULL the residual p - dequant(code) is written back into e.
 * codes: ceil(n*bits/8) bytes, or ceil(ceil(n/8)*W/8) with dense packing
 * (fully written, pad bits zero).
 * meta: nb * k floats.  tie: nb bytes or NULL (near-tie record). */
int gqref_quantize(int scheme, int d, int s, int L, int flags, float clip_sigma,
                   int64_t i0, int64_t n, const float *g, float *e,
                   uint64_t seed, uint32_t step,
                   uint8_t *codes, float *meta, uint8_t *tie);

/* Levels only (the meta part of gqref_quantize); e may be NULL. */
int gqref_select_levels(int scheme, int d, int s, int L, int flags,
                        float clip_sigma, int64_t i0, int64_t n,
                        const float *g, const float *e, float *meta,
                        uint8_t *tie);

/* xhat[i] = level value that code i stands for (flags: the payload's flags,
 * bit 1 = dense packing). */
int gqref_dequantize(int scheme, int d, int s, int L, int flags, int64_t n,
                     const uint8_t *codes, const float *meta, float *xhat);

/* e <- fl(fl(g + e) - xhat). */
int gqref_error_feedback(int scheme, int d, int s, int L, int flags, int64_t n,
                         const float *g, float *e,
                         const uint8_t *codes, const float *meta);

/* out <- fl32(beta*out + alpha*sum_w xhat_w), evaluated in binary64 and
 * rounded once; beta == 0 means out is not read. */
int gqref_dequantize_accumulate(int scheme, int d, int s, int L, int flags,
                                int64_t n, int W, const uint8_t *const *codes,
                                const float *const *meta, float alpha,
                                float beta, float *out);

/* Per-layer scale (TernGrad): the uniform scheme with layer l = elements
 * [off[l], off[l+1]) of the flat gradient as one bucket (off[0] = 0,
 * off[nl] = n, non-decreasing; empty layers allowed).  meta: nl floats
 * (each layer's max-abs).  flags: dense (bit 1) and nearest (bit 2); codes
 * as in gqref_quantize for the flat index. */
int gqref_quantize_layers(int s, int flags, int64_t n, int nl,
                          const int64_t *off, const float *g, float *e,
                          uint64_t seed, uint32_t step, uint8_t *codes,
                          float *meta);
int gqref_dequantize_accumulate_layers(int s, int flags, int64_t n, int nl,
                                       const int64_t *off, int W,
                                       const uint8_t *const *codes,
                                       const float *const *meta, float alpha,
                                       float beta, float *out);

/* Top-K sparsification with quantization: per bucket the min(K, n_j)
 * elements of largest |p| (ties: lower index) are rounded on the uniform
 * grid of s levels per sign; the rest count as 0 (the residual keeps them).
 * codes: nb records of gqref_topk_record_words(d, s, K) 32-bit words, slot t
 * = (index within the bucket: log2 d bits, code: b bits), LSB first.
 * meta: nb floats (max-abs).  flags: bit 2 (nearest) only. */
int gqref_topk_record_words(int d, int s, int K);
int gqref_quantize_topk(int d, int s, int K, int flags, int64_t n,
                        const float *g, float *e, uint64_t seed, uint32_t step,
                        uint8_t *codes, float *meta);
int gqref_dequantize_accumulate_topk(int d, int s, int K, int flags, int64_t n,
                                     int W, const uint8_t *const *codes,
                                     const float *const *meta, float alpha,
                                     float beta, float *out);

/* Dense packing (flags bit 1): groups of 8 codes as one base-A integer,
 * first code least significant, in fields of gqref_dense_width(A) =
 * ceil(log2(A^8)) bits of the LSB-first stream; A <= 16. */
int gqref_dense_width(int A);
void gqref_pack_dense(int A, int64_t n, const uint32_t *digits, uint8_t *codes);
void gqref_unpack_dense(int A, int64_t n, const uint8_t *codes, uint32_t *digits);

/* Raw bitstream access, element i of a stream with `bits` bits per code. */
void gqref_pack(int bits, int64_t n, const uint32_t *vals, uint8_t *codes);
void gqref_unpack(int bits, int64_t n, const uint8_t *codes, uint32_t *vals);

/* Elias gamma coding of uniform-scheme codes (QSGD's lossless integer
 * coding): code c -> gamma(|c| + 1), then a sign bit (1 = negative) when
 * c != 0; bucket records word-aligned; off: nb + 1 word offsets (off[0] = 0,
 * off[nb] = words used).  encode with words == NULL fills off only.
 * max_words: the stream size when every code has |c| = s. */
int64_t gqref_elias_max_words(int d, int s, int64_t n);
int gqref_elias_encode(int d, int s, int64_t n, const uint8_t *codes,
                       uint64_t *off, uint32_t *words);
int gqref_elias_decode(int d, int s, int64_t n, const uint64_t *off,
                       const uint32_t *words, uint8_t *codes);

void gqref_set_threads(int t);
int gqref_get_threads(void);

#ifdef __cplusplus
}
#endif
#endif
