/*
 * gqref.c — the CPU oracle.  TEST INFRASTRUCTURE ONLY (see gqref.h).
 *
 * Plain scalar C, one bucket at a time, OpenMP only across independent
 * buckets; nothing is blocked, fused or reordered beyond what the method
 * states.  Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp.
 *
 * Numerics: per-element arithmetic is IEEE binary32 with round-to-nearest
 * (x86-64 SSE, no contraction); sums that feed a decision or a mean
 * (means, RMS, prefix sums, split objectives, ORQ gains) are binary64 with
 * Neumaier compensation, in index or sorted order.
 */
#include "gqref.h"

#include <float.h>
#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

enum { UNIFORM = 0, BIN_SIGN = 1, BIN_OPT = 2, ORQ = 3 };
#define TIE_REL 1e-12

/* ------------------------------------------------------------------ RNG --
 * Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
 * Easy as 1, 2, 3" (SC'11).  Ten rounds of the 4x32 S-box with multipliers
 * 0xD2511F53 and 0xCD9E8D57, key schedule bumped by the Weyl constants
 * 0x9E3779B9 and 0xBB67AE85 between rounds.
 * The pages only ask for rounding that is random and unbiased ("Gradient
 * Quantization" glossary, Stochastic Quantization bullet); the generator and
 * its counter layout are this implementation's choice:
 *   key = (seed lo, seed hi), counter = (i/4 lo, i/4 hi, step, 0),
 *   element i uses output word i mod 4.
 */
void gqref_philox(uint64_t seed, uint64_t ctr, uint32_t step, uint32_t out[4]) {
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  uint32_t c0 = (uint32_t)ctr, c1 = (uint32_t)(ctr >> 32), c2 = step, c3 = 0;
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    uint64_t m0 = (uint64_t)0xD2511F53u * c0;
    uint64_t m1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t hi0 = (uint32_t)(m0 >> 32), lo0 = (uint32_t)m0;
    uint32_t hi1 = (uint32_t)(m1 >> 32), lo1 = (uint32_t)m1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

void gqref_philox_blocks(uint64_t seed, uint64_t ctr0, int64_t nblocks,
                         uint32_t step, uint32_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nblocks; ++b)
    gqref_philox(seed, ctr0 + (uint64_t)b, step, out + 4 * b);
}

/* u_i in [0, 1): the top 24 bits of element i's word, exact in binary32. */
static float uniform_u(uint64_t seed, uint32_t step, int64_t i) {
  uint32_t w[4];
  gqref_philox(seed, (uint64_t)i / 4u, step, w);
  return (float)(w[i % 4] >> 8) * 0x1p-24f;
}

/* ------------------------------------------------------------ packing --
 * One LSB-first bitstream: code i occupies stream bits [b*i, b*i + b),
 * stream bit t is bit (t mod 8) of byte t/8, code bit 0 first. */
static void put_code(uint8_t *codes, int64_t i, int bits, uint32_t v) {
  for (int t = 0; t < bits; ++t) {
    int64_t pos = i * bits + t;
    if ((v >> t) & 1u) codes[pos / 8] |= (uint8_t)(1u << (pos % 8));
  }
}

static uint32_t get_code(const uint8_t *codes, int64_t i, int bits) {
  uint32_t v = 0;
  for (int t = 0; t < bits; ++t) {
    int64_t pos = i * bits + t;
    v |= (uint32_t)((codes[pos / 8] >> (pos % 8)) & 1u) << t;
  }
  return v;
}

void gqref_pack(int bits, int64_t n, const uint32_t *vals, uint8_t *codes) {
  memset(codes, 0, (size_t)((n * bits + 7) / 8));
  for (int64_t i = 0; i < n; ++i) put_code(codes, i, bits, vals[i]);
}

void gqref_unpack(int bits, int64_t n, const uint8_t *codes, uint32_t *vals) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) vals[i] = get_code(codes, i, bits);
}

/* ------------------------------------------------------ dense packing --
 * An alphabet of A symbols (A <= 16) that is not a power of two wastes
 * bits in a fixed-width field.  Dense packing groups 8 consecutive codes
 * into one base-A integer V = sum_t digit(8g + t) * A^t (the first code is
 * the least significant digit; digits of absent elements are 0) and writes
 * V as a field of W = ceil(log2(A^8)) bits: field g occupies stream bits
 * [W*g, W*g + W), least significant bit first, in the same LSB-first
 * bitstream as fixed-width codes. */
int gqref_dense_width(int A) {
  if (A < 2 || A > 16) return -1;
  uint64_t p = 1;
  for (int i = 0; i < 8; ++i) p *= (uint64_t)A;
  int w = 0;
  while (((uint64_t)1 << w) < p) ++w;
  return w;
}

static void put_bits(uint8_t *codes, int64_t bit0, int w, uint64_t v) {
  for (int t = 0; t < w; ++t) {
    int64_t pos = bit0 + t;
    if ((v >> t) & 1u) codes[pos / 8] |= (uint8_t)(1u << (pos % 8));
  }
}

static uint64_t get_bits(const uint8_t *codes, int64_t bit0, int w) {
  uint64_t v = 0;
  for (int t = 0; t < w; ++t) {
    int64_t pos = bit0 + t;
    v |= (uint64_t)((codes[pos / 8] >> (pos % 8)) & 1u) << t;
  }
  return v;
}

/* Encode digits[0 .. n) (each < A) as dense fields starting at field 0. */
void gqref_pack_dense(int A, int64_t n, const uint32_t *digits, uint8_t *codes) {
  int w = gqref_dense_width(A);
  int64_t groups = (n + 7) / 8;
  memset(codes, 0, (size_t)((groups * w + 7) / 8));
  for (int64_t g = 0; g < groups; ++g) {
    uint64_t v = 0, place = 1;
    for (int t = 0; t < 8; ++t) {
      int64_t i = 8 * g + t;
      if (i < n) v += (uint64_t)digits[i] * place;
      place *= (uint64_t)A;
    }
    put_bits(codes, g * w, w, v);
  }
}

/* Digit of element i of a dense stream. */
static uint32_t dense_digit(const uint8_t *codes, int A, int w, int64_t i) {
  uint64_t v = get_bits(codes, (i / 8) * w, w);
  for (int64_t t = 0; t < i % 8; ++t) v /= (uint64_t)A;
  return (uint32_t)(v % (uint64_t)A);
}

void gqref_unpack_dense(int A, int64_t n, const uint8_t *codes, uint32_t *digits) {
  int w = gqref_dense_width(A);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) digits[i] = dense_digit(codes, A, w, i);
}

/* ---------------------------------------------------- compensated sums -- */
typedef struct {
  double s, c;
} nsum;

static void nadd(nsum *a, double x) {
  double t = a->s + x;
  if (fabs(a->s) >= fabs(x))
    a->c += (a->s - t) + x;
  else
    a->c += (x - t) + a->s;
  a->s = t;
}

static double nval(const nsum *a) { return a->s + a->c; }

/* ---------------------------------------------------------- parameters -- */
static int ceil_log2(int v) {
  int b = 0;
  while ((1 << b) < v) ++b;
  return b;
}

int gqref_bits(int scheme, int s, int L) {
  switch (scheme) {
    case UNIFORM: {
      /* codes -s..s in two's complement, widths 2, 3, 4 or 8 bits */
      if (s < 1 || s > 127) return -1;
      int w = ceil_log2(2 * s + 1);
      return w <= 4 ? w : 8;
    }
    case BIN_SIGN:
    case BIN_OPT:
      return 1;
    case ORQ:
      if (L < 2 || L > 16) return -1;
      return ceil_log2(L);
    default:
      return -1;
  }
}

int gqref_meta_per_bucket(int scheme, int L) {
  switch (scheme) {
    case UNIFORM:
      return 1;
    case BIN_SIGN:
    case BIN_OPT:
      return 2;
    case ORQ:
      return (L >= 2 && L <= 16) ? L : -1;
    default:
      return -1;
  }
}

static int check(int scheme, int d, int s, int L, int64_t i0, int64_t n) {
  if (n < 1 || i0 < 0) return -1;
  if (d < 64 || d > 32768 || (d & (d - 1))) return -1;
  if (i0 % d) return -1;
  if (gqref_bits(scheme, s, L) < 0) return -1;
  return 0;
}

/* Sign-extend a `bits`-wide two's-complement code. */
static int32_t sext(uint32_t v, int bits) {
  uint32_t m = 1u << (bits - 1);
  return (int32_t)((v ^ m) - m);
}

static int cmp_float(const void *a, const void *b) {
  float x = *(const float *)a, y = *(const float *)b;
  return (x > y) - (x < y);
}

/* Sorted copy of a bucket with -0.0 turned into +0.0. */
static float *sorted_copy(const float *p, int64_t nj) {
  float *y = (float *)malloc((size_t)nj * sizeof(float));
  for (int64_t t = 0; t < nj; ++t) y[t] = (p[t] == 0.0f) ? 0.0f : p[t];
  qsort(y, (size_t)nj, sizeof(float), cmp_float);
  return y;
}

/* ====================================================== level selection ==
 * Each selector fills the bucket's meta row (and the tie flag) from the
 * bucket's effective values p (n_j real elements, no padding). */

/* Uniform: the max-abs scale ("Gradient Quantization" glossary, core
 * mechanism: scale by the maximum absolute value). */
static void levels_uniform(const float *p, int64_t nj, float *meta) {
  float m = 0.0f;
  for (int64_t t = 0; t < nj; ++t) {
    float a = fabsf(p[t]);
    if (a > m) m = a;
  }
  meta[0] = m;
}

/* Sign split: codes 0 for p < 0, 1 for p >= 0; each level is the mean of its
 * side ("Gradient Quantization" glossary, ternary/binary paragraph: SignSGD
 * sends signs; the magnitudes are the side means). */
static void levels_sign(const float *p, int64_t nj, float *meta) {
  nsum neg = {0, 0}, pos = {0, 0};
  int64_t nn = 0, np = 0;
  for (int64_t t = 0; t < nj; ++t) {
    if (p[t] >= 0.0f) {
      nadd(&pos, (double)p[t]);
      ++np;
    } else {
      nadd(&neg, (double)p[t]);
      ++nn;
    }
  }
  meta[0] = nn ? (float)(nval(&neg) / (double)nn) : 0.0f;
  meta[1] = np ? (float)(nval(&pos) / (double)np) : 0.0f;
}

/* Two-level optimal split (BinGrad-b: the biased two-level quantizer whose
 * levels minimise the squared error; "Optimal Gradient Quantization
 * Condition" review, §Proposed method).  Plain definition: 1-D 2-means.
 * Its optimal clusters are contiguous in sorted order and each level is its
 * cluster's mean, so: sort, try every split k between distinct values,
 * maximise F(k) = P_k^2/k + Q_k^2/(n-k) (sum of squares minus SSE), take the
 * smallest k on exact equality.  Writes meta (a, b) and returns the threshold
 * y_k* (codes are p >= threshold); *no_split = 1 when every value is equal. */
static float levels_binopt(const float *p, int64_t nj, float *meta,
                           uint8_t *tie, int *no_split) {
  float *y = sorted_copy(p, nj);
  double *P = (double *)malloc((size_t)(nj + 1) * sizeof(double));
  double *Q = (double *)malloc((size_t)(nj + 1) * sizeof(double));
  nsum acc = {0, 0};
  P[0] = 0.0;
  for (int64_t t = 0; t < nj; ++t) {
    nadd(&acc, (double)y[t]);
    P[t + 1] = nval(&acc);
  }
  acc.s = acc.c = 0.0;
  Q[nj] = 0.0;
  for (int64_t t = nj - 1; t >= 0; --t) {
    nadd(&acc, (double)y[t]);
    Q[t] = nval(&acc);
  }
  int64_t kstar = -1;
  double best = -1.0;
  for (int64_t k = 1; k < nj; ++k) {
    if (!(y[k - 1] < y[k])) continue;
    double F = P[k] * P[k] / (double)k + Q[k] * Q[k] / (double)(nj - k);
    if (F > best) {
      best = F;
      kstar = k;
    }
  }
  float thr;
  if (kstar < 0) {
    meta[0] = meta[1] = y[0];
    *no_split = 1;
    thr = y[0];
    if (tie) *tie = 0;
  } else {
    double second = -1.0;
    for (int64_t k = 1; k < nj; ++k) {
      if (k == kstar || !(y[k - 1] < y[k])) continue;
      double F = P[k] * P[k] / (double)k + Q[k] * Q[k] / (double)(nj - k);
      if (F > second) second = F;
    }
    if (tie) *tie = (second >= best * (1.0 - TIE_REL)) ? 1 : 0;
    nsum lo = {0, 0}, hi = {0, 0};
    for (int64_t t = 0; t < kstar; ++t) nadd(&lo, (double)y[t]);
    for (int64_t t = kstar; t < nj; ++t) nadd(&hi, (double)y[t]);
    meta[0] = (float)(nval(&lo) / (double)kstar);
    meta[1] = (float)(nval(&hi) / (double)(nj - kstar));
    *no_split = 0;
    thr = y[kstar];
  }
  free(y);
  free(P);
  free(Q);
  return thr;
}

/* Symmetric clip at clip_sigma times the bucket's RMS ("Optimal Gradient
 * Quantization Condition" review, §Proposed method: clipping helps ORQ).
 * Returns C and flags a possible 1-ulp disagreement in the fp32 rounding of
 * clip_sigma*sigma (value within TIE_REL of a binary32 rounding midpoint). */
static float clip_bound(const float *p, int64_t nj, float clip_sigma,
                        uint8_t *tie) {
  nsum sq = {0, 0};
  for (int64_t t = 0; t < nj; ++t) nadd(&sq, (double)p[t] * (double)p[t]);
  double sigma = sqrt(nval(&sq) / (double)nj);
  double cd = (double)clip_sigma * sigma;
  float c = (float)cd;
  if (tie && cd > 0.0) {
    float lo = (double)c <= cd ? c : nextafterf(c, 0.0f);
    float hi = nextafterf(lo, INFINITY);
    double mid = 0.5 * ((double)lo + (double)hi);
    if (fabs(cd - mid) <= TIE_REL * cd) *tie = 1;
  }
  return c;
}

/* ORQ level selection ("Optimal Gradient Quantization Condition" review,
 * §Proposed method: multi-level unbiased quantization whose levels are
 * picked greedily to minimise the expected rounding variance).
 * With a value x rounded at random between adjacent levels a <= x <= b the
 * variance is (b-x)(x-a).  Start from {min, max} (every value must lie inside
 * the outer levels for the rounding to stay unbiased) and insert one level at
 * a time, the one that reduces the summed variance most.  Inserting c in
 * (a, b) reduces it by
 *     G(c) = (b-c) * sum_{a<y<=c} (y-a)  +  (c-a) * sum_{c<y<b} (b-y),
 * which is piecewise linear between data values, so the candidates are the
 * distinct data values strictly inside an interval.  Exact ties take the
 * smaller c; with fewer distinct values than levels the rest repeat max.
 * lev must hold L floats; y is the sorted bucket (n_j values). */
static void orq_greedy(const float *y, int64_t nj, int L, float *lev,
                       uint8_t *tie) {
  int cnt = 2;
  lev[0] = y[0];
  lev[1] = y[nj - 1];
  if (y[0] == y[nj - 1]) {
    for (int j = 0; j < L; ++j) lev[j] = y[0];
    return;
  }
  double *A = (double *)malloc((size_t)nj * sizeof(double));
  double *B = (double *)malloc((size_t)nj * sizeof(double));
  while (cnt < L) {
    double best = -1.0, second = -1.0;
    float bestc = 0.0f;
    int64_t lo = 0;
    for (int j = 0; j + 1 < cnt; ++j) {
      float a = lev[j], b = lev[j + 1];
      if (!(a < b)) continue;
      while (lo < nj && !(y[lo] > a)) ++lo;
      int64_t hi = lo;
      while (hi < nj && y[hi] < b) ++hi; /* interior values are y[lo..hi) */
      if (hi == lo) continue;
      nsum acc = {0, 0};
      for (int64_t t = lo; t < hi; ++t) {
        nadd(&acc, (double)y[t] - (double)a);
        A[t] = nval(&acc);
      }
      acc.s = acc.c = 0.0;
      for (int64_t t = hi - 1; t >= lo; --t) {
        B[t] = nval(&acc); /* sum over y[t+1 .. hi) */
        nadd(&acc, (double)b - (double)y[t]);
      }
      for (int64_t t = lo; t < hi; ++t) {
        if (t + 1 < hi && y[t + 1] == y[t]) continue; /* last of a run */
        double c = (double)y[t];
        double G = ((double)b - c) * A[t] + (c - (double)a) * B[t];
        if (G > best) {
          second = best;
          best = G;
          bestc = y[t];
        } else if (G > second) {
          second = G;
        }
      }
      lo = hi;
    }
    if (best < 0.0) {
      for (int j = cnt; j < L; ++j) lev[j] = y[nj - 1];
      break;
    }
    if (tie && second >= best * (1.0 - TIE_REL)) *tie = 1;
    int pos = cnt;
    while (pos > 0 && lev[pos - 1] > bestc) {
      lev[pos] = lev[pos - 1];
      --pos;
    }
    lev[pos] = bestc;
    ++cnt;
  }
  free(A);
  free(B);
}

/* ORQ levels by recursive bisection, the other reading of the greedy
 * selection that also yields the 3 / 5 / 9 levels of the review's
 * experiments (2^k + 1): rounds in which every interval between adjacent
 * levels receives its own best level c (the G(c) above, restricted to that
 * interval) at once.  When a full round would pass L levels, only the
 * round's candidates with the largest G are inserted (ties: smaller c).
 * Starts, degenerate buckets and the fill with max are as in orq_greedy.
 * The near-tie record covers the best and second-best candidate of each
 * interval, and in a partial round the last candidate taken and the first
 * left out. */
static void orq_bisect(const float *y, int64_t nj, int L, float *lev,
                       uint8_t *tie) {
  int cnt = 2;
  lev[0] = y[0];
  lev[1] = y[nj - 1];
  if (y[0] == y[nj - 1]) {
    for (int j = 0; j < L; ++j) lev[j] = y[0];
    return;
  }
  double *A = (double *)malloc((size_t)nj * sizeof(double));
  double *B = (double *)malloc((size_t)nj * sizeof(double));
  float cand[16];
  double gain[16];
  while (cnt < L) {
    int m = 0;
    int64_t lo = 0;
    for (int j = 0; j + 1 < cnt; ++j) {
      float a = lev[j], b = lev[j + 1];
      if (!(a < b)) continue;
      while (lo < nj && !(y[lo] > a)) ++lo;
      int64_t hi = lo;
      while (hi < nj && y[hi] < b) ++hi; /* interior values are y[lo..hi) */
      if (hi == lo) continue;
      nsum acc = {0, 0};
      for (int64_t t = lo; t < hi; ++t) {
        nadd(&acc, (double)y[t] - (double)a);
        A[t] = nval(&acc);
      }
      acc.s = acc.c = 0.0;
      for (int64_t t = hi - 1; t >= lo; --t) {
        B[t] = nval(&acc);
        nadd(&acc, (double)b - (double)y[t]);
      }
      double best = -1.0, second = -1.0;
      float bestc = 0.0f;
      for (int64_t t = lo; t < hi; ++t) {
        if (t + 1 < hi && y[t + 1] == y[t]) continue;
        double c = (double)y[t];
        double G = ((double)b - c) * A[t] + (c - (double)a) * B[t];
        if (G > best) {
          second = best;
          best = G;
          bestc = y[t];
        } else if (G > second) {
          second = G;
        }
      }
      if (tie && second >= best * (1.0 - TIE_REL)) *tie = 1;
      cand[m] = bestc;
      gain[m] = best;
      ++m;
      lo = hi;
    }
    if (m == 0) {
      for (int j = cnt; j < L; ++j) lev[j] = y[nj - 1];
      break;
    }
    int room = L - cnt;
    if (m > room) {
      /* keep the room largest gains; equal gains keep the smaller c.  The
       * candidates arrive in ascending c (intervals are visited in order),
       * and a stable insertion sort by decreasing gain keeps that order
       * among equal gains. */
      for (int a = 1; a < m; ++a) {
        double tg = gain[a];
        float tc = cand[a];
        int b = a;
        while (b > 0 && gain[b - 1] < tg) {
          gain[b] = gain[b - 1];
          cand[b] = cand[b - 1];
          --b;
        }
        gain[b] = tg;
        cand[b] = tc;
      }
      if (tie && gain[room] >= gain[room - 1] * (1.0 - TIE_REL)) *tie = 1;
      m = room;
    }
    for (int k = 0; k < m; ++k) {
      int pos = cnt;
      while (pos > 0 && lev[pos - 1] > cand[k]) {
        lev[pos] = lev[pos - 1];
        --pos;
      }
      lev[pos] = cand[k];
      ++cnt;
    }
  }
  free(A);
  free(B);
}

/* ========================================================== per bucket == */
typedef struct {
  int scheme, d, s, L, flags, bits, k;
  float clip_sigma;
  int dense, A, w; /* dense packing: alphabet size and field width */
  int nearest;     /* deterministic rounding to the nearest level */
} params;

/* Select the bucket's levels from its effective values p; for ORQ also
 * writes the clipped values into pc (if non-NULL) and returns them sorted
 * internally.  BIN_OPT returns its threshold through *thr. */
static void select_bucket(const params *pr, const float *p, int64_t nj,
                          float *meta, uint8_t *tie, float *pc, float *thr,
                          int *no_split) {
  if (tie) *tie = 0;
  switch (pr->scheme) {
    case UNIFORM:
      levels_uniform(p, nj, meta);
      break;
    case BIN_SIGN:
      levels_sign(p, nj, meta);
      break;
    case BIN_OPT:
      *thr = levels_binopt(p, nj, meta, tie, no_split);
      break;
    case ORQ: {
      float *v = pc ? pc : (float *)malloc((size_t)nj * sizeof(float));
      if (pr->flags & 1) {
        float c = clip_bound(p, nj, pr->clip_sigma, tie);
        for (int64_t t = 0; t < nj; ++t) v[t] = fminf(fmaxf(p[t], -c), c);
      } else {
        memcpy(v, p, (size_t)nj * sizeof(float));
      }
      float *y = sorted_copy(v, nj);
      if (pr->flags & 8) orq_bisect(y, nj, pr->L, meta, tie);
      else orq_greedy(y, nj, pr->L, meta, tie);
      free(y);
      if (!pc) free(v);
      break;
    }
  }
}

/* Level value for a code value c (signed integer -s..s for the uniform
 * scheme, level index otherwise), given the bucket's meta row. */
static float dequant_one(const params *pr, int32_t c, const float *meta) {
  switch (pr->scheme) {
    case UNIFORM: {
      /* step = M / s; xhat = c * step, each rounded once. */
      float delta = meta[0] / (float)pr->s;
      return (float)c * delta;
    }
    case BIN_SIGN:
    case BIN_OPT:
      return c ? meta[1] : meta[0];
    default:
      return meta[c];
  }
}

/* Code value of element i of a payload (fixed-width or dense). */
static int32_t read_code(const params *pr, const uint8_t *codes, int64_t i) {
  if (pr->dense) {
    int32_t digit = (int32_t)dense_digit(codes, pr->A, pr->w, i);
    return pr->scheme == UNIFORM ? digit - pr->s : digit;
  }
  uint32_t raw = get_code(codes, i, pr->bits);
  return pr->scheme == UNIFORM ? sext(raw, pr->bits) : (int32_t)raw;
}

/* Whether a value a fraction q of the way from its lower to its upper level
 * takes the upper one.  Random rounding: iff u < q, so with probability q
 * ("Gradient Quantization" glossary, Stochastic Quantization bullet).
 * Deterministic rounding (flags bit 2; same glossary, Deterministic
 * Quantization bullet: the nearest level): iff q > 1/2, an exact tie going
 * to the lower level. */
static int round_up(const params *pr, float q, float u) {
  return pr->nearest ? q > 0.5f : u < q;
}

/* Code for one element: random rounding between the two adjacent levels
 * ("Gradient Quantization" glossary, Stochastic Quantization bullet: a value
 * a fraction q of the way from the lower to the upper level rounds up with
 * probability q).  Rounds up iff u < q. */
static int32_t code_uniform(const params *pr, float p, float M, float u) {
  if (M == 0.0f || p == 0.0f) return 0;
  /* A bucket whose max-abs is tiny is scaled up by 2^96 first (exact), so
   * s/M stays finite; for every normal-range bucket the factor is 1. */
  float up = (M < 0x1p-96f) ? 0x1p96f : 1.0f;
  float inv = (float)pr->s / (M * up);
  float r = (fabsf(p) * up) * inv;
  if (r > (float)pr->s) r = (float)pr->s;
  float l = floorf(r);
  float q = r - l;
  int32_t mag = (int32_t)l + (round_up(pr, q, u) ? 1 : 0);
  return (p < 0.0f) ? -mag : mag;
}

static uint32_t code_orq(const params *pr, float pcl, const float *lev,
                         float u) {
  int L = pr->L;
  for (int j = 0; j < L; ++j)
    if (lev[j] == pcl) return (uint32_t)j;
  int j = 0;
  for (int t = 0; t < L; ++t)
    if (lev[t] < pcl) j = t;
  float num = pcl - lev[j];
  float den = lev[j + 1] - lev[j];
  float q = num / den;
  return (uint32_t)(j + (round_up(pr, q, u) ? 1 : 0));
}

static void quantize_bucket(const params *pr, int64_t gi, const float *g,
                            float *e, int64_t nj, uint64_t seed, uint32_t step,
                            uint8_t *codes, int64_t li, float *meta,
                            uint8_t *tie) {
  float *p = (float *)malloc((size_t)nj * sizeof(float));
  float *pc = (float *)malloc((size_t)nj * sizeof(float));
  int32_t *cv = (int32_t *)malloc((size_t)nj * sizeof(int32_t));
  /* Error feedback: add the carried residual before quantizing ("Gradient
   * Quantization" glossary, error-feedback paragraph). */
  for (int64_t t = 0; t < nj; ++t) p[t] = e ? g[t] + e[t] : g[t];
  float thr = 0.0f;
  int no_split = 0;
  select_bucket(pr, p, nj, meta, tie, pc, &thr, &no_split);
  for (int64_t t = 0; t < nj; ++t) {
    int32_t c;
    switch (pr->scheme) {
      case UNIFORM:
        c = code_uniform(pr, p[t], meta[0],
                         pr->nearest ? 0.0f : uniform_u(seed, step, gi + t));
        break;
      case BIN_SIGN:
        c = p[t] >= 0.0f ? 1 : 0;
        break;
      case BIN_OPT:
        c = no_split ? 0 : (p[t] >= thr ? 1 : 0);
        break;
      default:
        c = (int32_t)code_orq(pr, pc[t], meta,
                              pr->nearest ? 0.0f : uniform_u(seed, step, gi + t));
        break;
    }
    cv[t] = c;
    if (!pr->dense) put_code(codes, li + t, pr->bits, (uint32_t)c & ((1u << pr->bits) - 1u));
    /* Residual with the unclipped value, so a clipped excess is carried. */
    if (e) e[t] = p[t] - dequant_one(pr, c, meta);
  }
  if (pr->dense) {
    /* the bucket starts at a multiple of d (a multiple of 8) in the stream,
     * so its fields are whole; a partial last group pads with digit 0 */
    for (int64_t g0 = 0; g0 < nj; g0 += 8) {
      uint64_t v = 0, place = 1;
      for (int t = 0; t < 8; ++t) {
        if (g0 + t < nj) {
          int32_t digit = pr->scheme == UNIFORM ? cv[g0 + t] + pr->s : cv[g0 + t];
          v += (uint64_t)digit * place;
        }
        place *= (uint64_t)pr->A;
      }
      put_bits(codes, ((li + g0) / 8) * pr->w, pr->w, v);
    }
  }
  free(p);
  free(pc);
  free(cv);
}

static int make_params(params *pr, int scheme, int d, int s, int L, int flags,
                       float clip_sigma) {
  pr->scheme = scheme;
  pr->d = d;
  pr->s = s;
  pr->L = L;
  pr->flags = flags;
  pr->clip_sigma = clip_sigma;
  pr->bits = gqref_bits(scheme, s, L);
  pr->k = gqref_meta_per_bucket(scheme, L);
  if (pr->bits < 0 || pr->k < 0) return -1;
  pr->dense = (flags & 2) ? 1 : 0;
  pr->nearest = (flags & 4) ? 1 : 0;
  if (pr->nearest && scheme != UNIFORM && scheme != ORQ) return -1;
  if ((flags & 8) && scheme != ORQ) return -1; /* bisection: ORQ only */
  pr->A = scheme == UNIFORM ? 2 * s + 1 : (scheme == ORQ ? L : 2);
  pr->w = pr->dense ? gqref_dense_width(pr->A) : 0;
  if (pr->dense && pr->w < 0) return -1;
  return 0;
}

/* Bytes of the code stream for n elements. */
static int64_t stream_bytes(const params *pr, int64_t n) {
  if (pr->dense) return (((n + 7) / 8) * pr->w + 7) / 8;
  return (n * pr->bits + 7) / 8;
}

int gqref_quantize(int scheme, int d, int s, int L, int flags, float clip_sigma,
                   int64_t i0, int64_t n, const float *g, float *e,
                   uint64_t seed, uint32_t step, uint8_t *codes, float *meta,
                   uint8_t *tie) {
  params pr;
  if (check(scheme, d, s, L, i0, n) || make_params(&pr, scheme, d, s, L, flags,
                                                   clip_sigma))
    return -1;
  if (!g || !codes || !meta) return -1;
  int64_t nb = (n + d - 1) / d;
  memset(codes, 0, (size_t)stream_bytes(&pr, n));
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < nb; ++j) {
    int64_t lo = j * d, nj = (n - lo < d) ? n - lo : d;
    quantize_bucket(&pr, i0 + lo, g + lo, e ? e + lo : NULL, nj, seed, step,
                    codes, lo, meta + j * pr.k, tie ? tie + j : NULL);
  }
  return 0;
}

int gqref_select_levels(int scheme, int d, int s, int L, int flags,
                        float clip_sigma, int64_t i0, int64_t n,
                        const float *g, const float *e, float *meta,
                        uint8_t *tie) {
  params pr;
  if (check(scheme, d, s, L, i0, n) || make_params(&pr, scheme, d, s, L, flags,
                                                   clip_sigma))
    return -1;
  if (!g || !meta) return -1;
  int64_t nb = (n + d - 1) / d;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < nb; ++j) {
    int64_t lo = j * d, nj = (n - lo < d) ? n - lo : d;
    float *p = (float *)malloc((size_t)nj * sizeof(float));
    for (int64_t t = 0; t < nj; ++t) p[t] = e ? g[lo + t] + e[lo + t] : g[lo + t];
    float thr;
    int no_split;
    select_bucket(&pr, p, nj, meta + j * pr.k, tie ? tie + j : NULL, NULL, &thr,
                  &no_split);
    free(p);
  }
  return 0;
}

int gqref_dequantize(int scheme, int d, int s, int L, int flags, int64_t n,
                     const uint8_t *codes, const float *meta, float *xhat) {
  params pr;
  if (check(scheme, d, s, L, 0, n) || make_params(&pr, scheme, d, s, L, flags, 0.f))
    return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    xhat[i] = dequant_one(&pr, read_code(&pr, codes, i), meta + (i / d) * pr.k);
  return 0;
}

int gqref_error_feedback(int scheme, int d, int s, int L, int flags, int64_t n,
                         const float *g, float *e, const uint8_t *codes,
                         const float *meta) {
  params pr;
  if (check(scheme, d, s, L, 0, n) || make_params(&pr, scheme, d, s, L, flags, 0.f))
    return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    float p = g[i] + e[i];
    e[i] = p - dequant_one(&pr, read_code(&pr, codes, i), meta + (i / d) * pr.k);
  }
  return 0;
}

int gqref_dequantize_accumulate(int scheme, int d, int s, int L, int flags,
                                int64_t n, int W, const uint8_t *const *codes,
                                const float *const *meta, float alpha,
                                float beta, float *out) {
  params pr;
  if (check(scheme, d, s, L, 0, n) || make_params(&pr, scheme, d, s, L, flags, 0.f))
    return -1;
  if (W < 1) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    nsum acc = {0, 0};
    for (int w = 0; w < W; ++w)
      nadd(&acc, (double)dequant_one(&pr, read_code(&pr, codes[w], i),
                                     meta[w] + (i / d) * pr.k));
    double v = (double)alpha * nval(&acc);
    if (beta != 0.0f) v += (double)beta * (double)out[i];
    out[i] = (float)v;
  }
  return 0;
}

/* ------------------------------------------------------ per-layer scale --
 * TernGrad's layout ("Gradient Quantization" glossary, ternary paragraph:
 * one scaling factor per layer): the flat gradient is the concatenation of
 * nl layers, layer l = elements [off[l], off[l+1]), and each layer is one
 * bucket of the uniform scheme, whatever its size or offset.  The random
 * counter is the element's index in the flat gradient and the codes form
 * the same flat stream as the bucketed layout (dense: 8-code fields by flat
 * index, so a field may hold codes of two layers).  meta[l] = the layer's
 * max-abs (0 for an empty layer). */
static int check_layers(int s, int flags, int64_t n, int nl,
                        const int64_t *off) {
  if (n < 1 || nl < 1 || !off) return -1;
  if (gqref_bits(UNIFORM, s, 2) < 0) return -1;
  if (flags & 1) return -1; /* clipping is an ORQ option */
  if (off[0] != 0 || off[nl] != n) return -1;
  for (int l = 0; l < nl; ++l)
    if (off[l + 1] < off[l]) return -1;
  return 0;
}

int gqref_quantize_layers(int s, int flags, int64_t n, int nl,
                          const int64_t *off, const float *g, float *e,
                          uint64_t seed, uint32_t step, uint8_t *codes,
                          float *meta) {
  params pr;
  if (check_layers(s, flags, n, nl, off) ||
      make_params(&pr, UNIFORM, 64, s, 2, flags, 0.f))
    return -1;
  if (!g || !codes || !meta) return -1;
  int32_t *cv = (int32_t *)malloc((size_t)n * sizeof(int32_t));
  if (!cv) return -1;
#pragma omp parallel for schedule(dynamic)
  for (int l = 0; l < nl; ++l) {
    int64_t lo = off[l], hi = off[l + 1];
    /* error feedback: p = g + e, then the layer's max-abs */
    float M = 0.0f;
    for (int64_t i = lo; i < hi; ++i) {
      float p = e ? g[i] + e[i] : g[i];
      if (fabsf(p) > M) M = fabsf(p);
    }
    meta[l] = M;
    for (int64_t i = lo; i < hi; ++i) {
      float p = e ? g[i] + e[i] : g[i];
      int32_t c = code_uniform(&pr, p, M, pr.nearest ? 0.0f : uniform_u(seed, step, i));
      cv[i] = c;
      if (e) e[i] = p - dequant_one(&pr, c, meta + l);
    }
  }
  /* pack the flat stream (sequentially: fields may straddle layers) */
  memset(codes, 0, (size_t)stream_bytes(&pr, n));
  if (pr.dense) {
    for (int64_t g0 = 0; g0 < n; g0 += 8) {
      uint64_t v = 0, place = 1;
      for (int t = 0; t < 8; ++t) {
        if (g0 + t < n) v += (uint64_t)(cv[g0 + t] + pr.s) * place;
        place *= (uint64_t)pr.A;
      }
      put_bits(codes, (g0 / 8) * pr.w, pr.w, v);
    }
  } else {
    for (int64_t i = 0; i < n; ++i)
      put_code(codes, i, pr.bits, (uint32_t)cv[i] & ((1u << pr.bits) - 1u));
  }
  free(cv);
  return 0;
}

int gqref_dequantize_accumulate_layers(int s, int flags, int64_t n, int nl,
                                       const int64_t *off, int W,
                                       const uint8_t *const *codes,
                                       const float *const *meta, float alpha,
                                       float beta, float *out) {
  params pr;
  if (check_layers(s, flags, n, nl, off) ||
      make_params(&pr, UNIFORM, 64, s, 2, flags, 0.f))
    return -1;
  if (W < 1) return -1;
#pragma omp parallel for schedule(dynamic)
  for (int l = 0; l < nl; ++l) {
    for (int64_t i = off[l]; i < off[l + 1]; ++i) {
      nsum acc = {0, 0};
      for (int w = 0; w < W; ++w)
        nadd(&acc, (double)dequant_one(&pr, read_code(&pr, codes[w], i),
                                       meta[w] + l));
      double v = (double)alpha * nval(&acc);
      if (beta != 0.0f) v += (double)beta * (double)out[i];
      out[i] = (float)v;
    }
  }
  return 0;
}

/* --------------------------------------------------------------- top-k --
 * Top-K sparsification combined with quantization ("gradient quantization
 * for communication" glossary, §Quantization Schemes: send only the largest
 * gradients, combined with quantization; error feedback keeps the rest).
 * Per bucket j (n_j real elements) the k_j = min(K, n_j) elements of largest
 * |p| are sent (equal magnitudes: the lower index first); their values are
 * rounded on the bucket's uniform grid exactly as gqref_quantize does for
 * the uniform scheme (M_j = max |p|, s levels per sign, u of the element's
 * flat index), the others count as 0.  Payload: meta[j] = M_j; codes: a
 * record of R = ceil(K (ib + b) / 32) 32-bit words per bucket (ib = log2 d
 * index bits, b the uniform code width), record j at byte 4 R j; slot t
 * (the kept elements in increasing index) holds the index within the
 * bucket, then the code (two's complement), LSB first from bit t (ib + b);
 * unused slots and pad bits are 0. */
int gqref_topk_record_words(int d, int s, int K) {
  int b = gqref_bits(UNIFORM, s, 2);
  if (b < 0 || d < 64 || (d & (d - 1)) || K < 1 || K > d) return -1;
  int ib = ceil_log2(d);
  return (int)(((int64_t)K * (ib + b) + 31) / 32);
}

typedef struct {
  float a;
  int64_t i;
} mag_idx;

static int by_mag_then_index(const void *x, const void *y) {
  const mag_idx *p = (const mag_idx *)x, *q = (const mag_idx *)y;
  if (p->a > q->a) return -1;
  if (p->a < q->a) return 1;
  return (p->i > q->i) - (p->i < q->i);
}

int gqref_quantize_topk(int d, int s, int K, int flags, int64_t n,
                        const float *g, float *e, uint64_t seed, uint32_t step,
                        uint8_t *codes, float *meta) {
  params pr;
  int R = gqref_topk_record_words(d, s, K);
  if (R < 0 || n < 1 || (flags & ~4) || !g || !codes || !meta) return -1;
  if (make_params(&pr, UNIFORM, d, s, 2, flags, 0.f)) return -1;
  int ib = ceil_log2(d), b = pr.bits;
  int64_t nb = (n + d - 1) / d;
  memset(codes, 0, (size_t)(nb * R * 4));
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < nb; ++j) {
    int64_t lo = j * d, nj = (n - lo < d) ? n - lo : d;
    int64_t k = nj < K ? nj : K;
    float *p = (float *)malloc((size_t)nj * sizeof(float));
    mag_idx *o = (mag_idx *)malloc((size_t)nj * sizeof(mag_idx));
    uint8_t *keep = (uint8_t *)calloc((size_t)nj, 1);
    float M = 0.0f;
    for (int64_t t = 0; t < nj; ++t) {
      p[t] = e ? g[lo + t] + e[lo + t] : g[lo + t];
      o[t].a = fabsf(p[t]);
      o[t].i = t;
      if (o[t].a > M) M = o[t].a;
    }
    meta[j] = M;
    qsort(o, (size_t)nj, sizeof(mag_idx), by_mag_then_index);
    for (int64_t t = 0; t < k; ++t) keep[o[t].i] = 1;
    uint8_t *rec = codes + (size_t)j * R * 4;
    int64_t slot = 0;
    for (int64_t t = 0; t < nj; ++t) {
      float xh = 0.0f;
      if (keep[t]) {
        int32_t c = code_uniform(&pr, p[t], M,
                                 pr.nearest ? 0.0f : uniform_u(seed, step, lo + t));
        uint64_t field = (uint64_t)t | ((uint64_t)((uint32_t)c & ((1u << b) - 1u)) << ib);
        put_bits(rec, slot * (ib + b), ib + b, field);
        ++slot;
        xh = dequant_one(&pr, c, meta + j);
      }
      if (e) e[lo + t] = p[t] - xh;
    }
    free(p);
    free(o);
    free(keep);
  }
  return 0;
}

int gqref_dequantize_accumulate_topk(int d, int s, int K, int flags, int64_t n,
                                     int W, const uint8_t *const *codes,
                                     const float *const *meta, float alpha,
                                     float beta, float *out) {
  params pr;
  int R = gqref_topk_record_words(d, s, K);
  if (R < 0 || n < 1 || W < 1 || (flags & ~4)) return -1;
  if (make_params(&pr, UNIFORM, d, s, 2, flags, 0.f)) return -1;
  int ib = ceil_log2(d), b = pr.bits;
  int64_t nb = (n + d - 1) / d;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < nb; ++j) {
    int64_t lo = j * d, nj = (n - lo < d) ? n - lo : d;
    int64_t k = nj < K ? nj : K;
    nsum *acc = (nsum *)calloc((size_t)nj, sizeof(nsum));
    for (int w = 0; w < W; ++w) {
      const uint8_t *rec = codes[w] + (size_t)j * R * 4;
      for (int64_t t = 0; t < k; ++t) {
        uint64_t field = get_bits(rec, t * (ib + b), ib + b);
        int64_t idx = (int64_t)(field & ((1u << ib) - 1u));
        int32_t c = sext((uint32_t)(field >> ib), b);
        if (idx < nj) nadd(&acc[idx], (double)dequant_one(&pr, c, meta[w] + j));
      }
    }
    for (int64_t t = 0; t < nj; ++t) {
      double v = (double)alpha * nval(&acc[t]);
      if (beta != 0.0f) v += (double)beta * (double)out[lo + t];
      out[lo + t] = (float)v;
    }
    free(acc);
  }
  return 0;
}

/* ------------------------------------------------ Elias gamma coding --
 * QSGD compresses its quantized integers further with Elias integer coding
 * ("Gradient Quantization" glossary, QSGD paragraph).  Reading: every code c
 * of the uniform scheme, in element order, becomes the Elias gamma code of
 * the positive integer m = |c| + 1 (floor(log2 m) zero bits, then the
 * floor(log2 m) + 1 binary digits of m, most significant first), followed by
 * one sign bit (1 = negative) when c != 0.  Each bucket's record starts on a
 * 32-bit word boundary (pad bits 0); off[j] is the first word of bucket j's
 * record, off[nb] the stream's word count.  Stream bit t of a record is bit
 * t mod 32 of its word t / 32.  Codes must lie in [-s, s]. */
static void word_put_bit(uint32_t *w, int64_t t, int bit) {
  if (bit) w[t / 32] |= 1u << (t % 32);
}

static int word_get_bit(const uint32_t *w, int64_t t) {
  return (int)((w[t / 32] >> (t % 32)) & 1u);
}

static int floor_log2_u(uint32_t m) {
  int L = 0;
  while ((m >> (L + 1)) != 0) ++L;
  return L;
}

static int64_t gamma_bits(int32_t c) {
  uint32_t m = (uint32_t)(c < 0 ? -c : c) + 1u;
  return 2 * floor_log2_u(m) + 1 + (c != 0);
}

int64_t gqref_elias_max_words(int d, int s, int64_t n) {
  if (d < 64 || (d & (d - 1)) || s < 1 || s > 127 || n < 1) return -1;
  int64_t worst = gamma_bits(s), nb = (n + d - 1) / d, tot = 0;
  for (int64_t j = 0; j < nb; ++j) {
    int64_t nj = (n - j * d < d) ? n - j * d : d;
    tot += (nj * worst + 31) / 32;
  }
  return tot;
}

int gqref_elias_encode(int d, int s, int64_t n, const uint8_t *codes,
                       uint64_t *off, uint32_t *words) {
  int b = gqref_bits(UNIFORM, s, 2);
  if (b < 0 || d < 64 || (d & (d - 1)) || n < 1 || !codes || !off) return -1;
  int64_t nb = (n + d - 1) / d;
  int bad = 0;
  /* each record's length, then the word offsets as their running sum */
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t j = 0; j < nb; ++j) {
    int64_t nj = (n - j * d < d) ? n - j * d : d, bits = 0;
    for (int64_t t = 0; t < nj; ++t) {
      int32_t c = sext(get_code(codes, j * d + t, b), b);
      if (c < -s || c > s) bad = 1;
      bits += gamma_bits(c);
    }
    off[j + 1] = (uint64_t)((bits + 31) / 32);
  }
  if (bad) return -1;
  off[0] = 0;
  for (int64_t j = 0; j < nb; ++j) off[j + 1] += off[j];
  if (!words) return 0;
  memset(words, 0, (size_t)off[nb] * 4);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < nb; ++j) {
    int64_t nj = (n - j * d < d) ? n - j * d : d;
    uint32_t *rec = words + off[j];
    int64_t t = 0;  /* bit cursor in the record */
    for (int64_t i = 0; i < nj; ++i) {
      int32_t c = sext(get_code(codes, j * d + i, b), b);
      uint32_t m = (uint32_t)(c < 0 ? -c : c) + 1u;
      int L = floor_log2_u(m);
      for (int k = 0; k < L; ++k) word_put_bit(rec, t++, 0);
      for (int k = L; k >= 0; --k) word_put_bit(rec, t++, (int)((m >> k) & 1u));
      if (c != 0) word_put_bit(rec, t++, c < 0);
    }
  }
  return 0;
}

static int decode_record(const uint32_t *rec, int64_t tmax, int64_t nj, int b,
                         int s, int64_t e0, uint8_t *codes) {
  int64_t t = 0;
  for (int64_t i = 0; i < nj; ++i) {
    int L = 0;
    while (t < tmax && word_get_bit(rec, t) == 0) { ++L; ++t; }
    if (L > 7 || t + L + 1 > tmax) return -1;  /* |c| + 1 <= 128 */
    uint32_t m = 0;
    for (int k = 0; k <= L; ++k) m = (m << 1) | (uint32_t)word_get_bit(rec, t++);
    int32_t c = (int32_t)(m - 1u);
    if (c > s) return -1;
    if (c != 0) {
      if (t >= tmax) return -1;
      if (word_get_bit(rec, t++)) c = -c;
    }
    put_code(codes, e0 + i, b, (uint32_t)c & ((1u << b) - 1u));
  }
  return 0;
}

int gqref_elias_decode(int d, int s, int64_t n, const uint64_t *off,
                       const uint32_t *words, uint8_t *codes) {
  int b = gqref_bits(UNIFORM, s, 2);
  if (b < 0 || d < 64 || (d & (d - 1)) || n < 1 || !off || !words || !codes)
    return -1;
  int64_t nb = (n + d - 1) / d;
  for (int64_t j = 0; j < nb; ++j)
    if (off[j + 1] < off[j]) return -1;
  memset(codes, 0, (size_t)((n * b + 7) / 8));
  int bad = 0;
  /* buckets own whole bytes of codes (d * b is a multiple of 8) */
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t j = 0; j < nb; ++j) {
    int64_t nj = (n - j * d < d) ? n - j * d : d;
    if (decode_record(words + off[j], 32 * (int64_t)(off[j + 1] - off[j]), nj,
                      b, s, j * d, codes))
      bad = 1;
  }
  return bad ? -1 : 0;
}

void gqref_set_threads(int t) {
  if (t > 0) omp_set_num_threads(t);
}

int gqref_get_threads(void) { return omp_get_max_threads(); }
