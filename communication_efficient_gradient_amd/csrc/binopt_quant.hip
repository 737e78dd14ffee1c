// binopt_quant.hip — BinGrad-b (the two-level quantizer whose levels
// minimise the squared error: the exact 1-D 2-means split of each bucket;
// "Optimal Gradient Quantization Condition" review, §Proposed method) with
// error feedback, for buckets of 1024 and more, without sorting the bucket.
//
// The split that maximises F(k) = P_k^2 / k + (S - P_k)^2 / (n - k) (P_k the
// sum of the k smallest values, S the bucket sum; the squared error is
// sum(y^2) - F) is found by bounding F over groups of candidate splits.  One
// workgroup owns a bucket, 16 or 32 values per thread, held as order-preserving
// integer keys of the canonical values:
//
//   1. Levels of refinement.  Each level cuts the candidate key ranges (at
//      most two; the first level one range, [min, max]) into 64 bins of equal
//      width in key space (so a bin is a run of consecutive sorted values, and
//      its value bounds lo, hi are exact floats).  Every thread adds its
//      values into the 64-bin (count, sum) histogram in LDS with one 64-bit
//      integer atomic per value (count in the high bits, the value in fixed
//      point below: exact, order-independent and, on this GPU, over 20x
//      cheaper than fp32 LDS atomics), each bin split into 16 columns by
//      lane so that few lanes of a wave meet on one address.  Prefix sums
//      give, at every bin edge, the split position K and the (quantized)
//      sum P of the values below it.
//   2. Bounds.  F at every bin edge is a lower bound LB of the optimum.  For
//      the splits inside a bin, (k, P_k) lies in the parallelogram between
//      the lines of slope lo and hi from the bin's first edge and into its
//      last edge; F is jointly convex in (k, P), so its maximum over the
//      parallelogram (clipped to 0 < k < n) is at a vertex.  A bin whose
//      upper bound stays below LB by more than the quantization of the sums
//      allows cannot hold the optimum and is dropped.  The surviving bins form
//      at most two new ranges: with survivors in both previous ranges the
//      hull of each, else the first run of surviving bins and the hull of the
//      rest.  The first wave evaluates the bins (lane b: bin b) and passes
//      the new ranges to the others through LDS.
//   3. When the surviving ranges hold at most 64 values, those values are
//      gathered, sorted by the first wave, and F is evaluated exactly (fp64
//      sums of the values below each range, fp64 prefix sums inside) at every
//      split between distinct values in or at the edges of the ranges; the
//      largest F wins, the smaller split on equality.
//   4. Codes [p >= y_k*] (compared in key space), the levels as the two
//      cluster means, the residual p - x_hat; the bucket is read once.
//
// A bucket whose candidates do not shrink to 64 values within ten levels
// (many equal values, whose splits the bounds cannot tell apart), or whose
// scale leaves the fixed-point range, is marked with NaN levels
// and left untouched; the caller then runs the sort-based kernel over the
// marked buckets only.
#include <type_traits>

#include "common.hpp"

namespace gq {
namespace {

constexpr int kBins = 64;     // bins per level (one per lane of the first wave)
constexpr int kCols = 16;     // LDS columns per bin (lane mod 16)
constexpr int kCap = 64;      // values the exact stage sorts (one per lane)
constexpr int kCapW = 256;    // ... when the levels run out (four per lane)
constexpr int kLevels = 10;   // levels before a bucket falls back to the sort
constexpr int kRow = kCols + 2;  // LDS words per bin row (padded)
// values per thread: 32 (workgroups of 64 to 512 threads), 16 at d = 1024
// (one wave), 64 at d = 32768 (512 threads, 32 of the keys in registers and
// 32 in LDS: two workgroups per CU, so one bucket's single-wave phases, its
// load and its stores overlap the other's work; with 1024 threads and all
// keys in registers a CU held one workgroup).  Every instance fits in 128
// VGPRs without spilling (four waves per SIMD).
__host__ __device__ constexpr int elems_per_thread(int d) {
  return d == 1024 ? 16 : (d == 32768 ? 64 : 32);
}
// held keys in registers (the rest in LDS)
__host__ __device__ constexpr int keys_in_regs(int d) {
  return elems_per_thread(d) < 32 ? elems_per_thread(d) : 32;
}

// Order-preserving key of a canonical fp32 value (no -0) and its inverse.
__device__ __forceinline__ uint32_t fkey(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float funkey(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// The value of a held key, recomputed where it is used: the empty asm hides
// that the key is loop-invariant, so the compiler does not keep a second
// register array of values across the refinement loop.
__device__ __forceinline__ float kval(uint32_t k) {
  asm volatile("" : "+v"(k));
  return funkey(k);
}

// A held key as an opaque value: the two passes over the keys in the exact
// stage recompute their range tests instead of keeping one predicate per
// key alive between them.
__device__ __forceinline__ uint32_t opaque(uint32_t k) {
  asm volatile("" : "+v"(k));
  return k;
}

// F at split k with P the sum below it (bounds: reciprocals refined by one
// Newton step, accurate to a few units in the last place).
__device__ __forceinline__ double obj_fast(double P, double k, double S, double n) {
  const double Q = S - P;
  double r1 = __builtin_amdgcn_rcp(k);
  r1 = __builtin_fma(r1, __builtin_fma(-k, r1, 1.0), r1);
  double r2 = __builtin_amdgcn_rcp(n - k);
  r2 = __builtin_fma(r2, __builtin_fma(-(n - k), r2, 1.0), r2);
  return P * P * r1 + Q * Q * r2;
}

// F with IEEE divisions, for the exact stage.
__device__ __forceinline__ double obj_exact(double P, double k, double S, double n) {
  const double Q = S - P;
  return P * P / k + Q * Q / (n - k);
}

template <int G>
__device__ __forceinline__ uint32_t group_min_u(uint32_t v) {
  return group_reduce<G>(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
template <int G>
__device__ __forceinline__ uint32_t group_max_u(uint32_t v) {
  return group_reduce<G>(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
template <int G>
__device__ __forceinline__ double group_sum_d(double v) {
  return group_reduce<G>(v, [](double a, double b) { return a + b; });
}
template <int G>
__device__ __forceinline__ double group_max_d(double v) {
  return group_reduce<G>(v, [](double a, double b) { return a > b ? a : b; });
}

// Group argmax of (value, key): larger value, then smaller key.
template <int G>
__device__ __forceinline__ void group_argmax_dk(double& v, int& key) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) {
    const double v2 = xshfl(v, o);
    const int k2 = xshfl(key, o);
    if (v2 > v || (v2 == v && k2 < key)) {
      v = v2;
      key = k2;
    }
  }
}

// Sort of the kCap = G * E2 values a group holds E2 per lane (lane t:
// positions t E2 .. t E2 + E2 - 1), ascending, bitonic in flip form: merge
// level K compares position i with i ^ (K - 1), then with i ^ J for
// J = K/4, ..., 1, the smaller value to the lower position.  Partners in the
// same lane: register compare-exchanges; in another lane: one lane exchange
// and one median of three (med3(a, b, -inf) = min, med3(a, b, +inf) = max).
template <int E2, int MASK, bool MIRROR>
__device__ __forceinline__ void sv_stage(float (&y)[E2], int t) {
  constexpr int TOP = MIRROR ? (MASK + 1) / 2 : MASK;
  if constexpr (MASK < E2) {
#pragma unroll
    for (int r = 0; r < E2; ++r) {
      const int r2 = r ^ MASK;
      if (r2 > r) {
        const float a = y[r], b = y[r2];
        y[r] = fminf(a, b);
        y[r2] = fmaxf(a, b);
      }
    }
  } else {
    constexpr int LM = MASK / E2;
    const float sel = (t & (TOP / E2)) == 0 ? -__builtin_inff() : __builtin_inff();
    float o[E2];
#pragma unroll
    for (int r = 0; r < E2; ++r) o[r] = xshfl(y[MIRROR ? E2 - 1 - r : r], LM);
#pragma unroll
    for (int r = 0; r < E2; ++r) y[r] = __builtin_amdgcn_fmed3f(y[r], o[r], sel);
  }
}

template <int E2, int K, int J>
__device__ __forceinline__ void sv_halves(float (&y)[E2], int t) {
  if constexpr (J >= 1) {
    sv_stage<E2, J, false>(y, t);
    sv_halves<E2, K, J / 2>(y, t);
  }
}

template <int E2, int N, int K>
__device__ __forceinline__ void sv_levels(float (&y)[E2], int t) {
  sv_stage<E2, K - 1, true>(y, t);
  sv_halves<E2, K, K / 4>(y, t);
  if constexpr (K < N) sv_levels<E2, N, 2 * K>(y, t);
}

template <int G>
__device__ __forceinline__ uint64_t group_lanes(int grp) {
  if constexpr (G == 64) return ~0ull;
  else return ((1ull << G) - 1ull) << (grp * G);
}

// Value of the lane N places lower in the same 16-lane row (0 in the row's
// first N lanes): one DPP move, no LDS.
template <int N>
__device__ __forceinline__ int row_shr(int v) {
  // every lane written (bound_ctrl zero-fills the first N of a row)
  return __builtin_amdgcn_mov_dpp(v, 0x110 + N, 0xF, 0xF, true);
}
template <int N>
__device__ __forceinline__ double row_shr(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)row_shr<N>((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)row_shr<N>((int)(uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Last lane of the previous row (rows 1 and 3 for BC = 15; rows 2 and 3
// take lane 31 for BC = 31), 0 in the other rows.
template <int BC>
__device__ __forceinline__ double row_bcast(double v) {
  constexpr int ctrl = BC == 15 ? 0x142 : 0x143;
  constexpr int rows = BC == 15 ? 0xA : 0xC;
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, ctrl, rows, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), ctrl, rows, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <int BC>
__device__ __forceinline__ int row_bcast(int v) {
  return __builtin_amdgcn_update_dpp(0, v, BC == 15 ? 0x142 : 0x143,
                                     BC == 15 ? 0xA : 0xC, 0xF, false);
}
template <int BC>
__device__ __forceinline__ long long row_bcast(long long v) {
  return __double_as_longlong(row_bcast<BC>(__longlong_as_double(v)));
}

template <int N>
__device__ __forceinline__ long long row_shr(long long v) {
  return __double_as_longlong(row_shr<N>(__longlong_as_double(v)));
}

// Inclusive prefix over the G lanes of a group (G = 16, 32, 64).
template <int G>
__device__ __forceinline__ double group_inclusive(double v) {
  v = v + row_shr<1>(v);
  v = v + row_shr<2>(v);
  v = v + row_shr<4>(v);
  v = v + row_shr<8>(v);
  if constexpr (G >= 32) v = v + row_bcast<15>(v);
  if constexpr (G >= 64) v = v + row_bcast<31>(v);
  return v;
}

// Inclusive prefix over the 64 lanes of a wave (DPP row shifts, then the
// row broadcasts).
template <typename V>
__device__ __forceinline__ V wave_inclusive(V v) {
  v = v + row_shr<1>(v);
  v = v + row_shr<2>(v);
  v = v + row_shr<4>(v);
  v = v + row_shr<8>(v);
  v = v + row_bcast<15>(v);
  v = v + row_bcast<31>(v);
  return v;
}

// A 64-bit value of lane `idx` (wave-uniform) in every lane.
__device__ __forceinline__ long long readlane64(long long v, int idx) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, idx);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), idx);
  return (long long)(((uint64_t)hi << 32) | lo);
}

template <int G>
__device__ __forceinline__ int group_min_i(int v) {
  return group_reduce<G>(v, [](int a, int b) { return a < b ? a : b; });
}

// Key of a raw fp32 bit pattern with -0 folded onto +0 (keys of finite
// values lie in [0x00800000, 0xff7fffff]).
__device__ __forceinline__ uint32_t canon_key(uint32_t b, bool negz) {
  const uint32_t k = b ^ ((uint32_t)((int)b >> 31) | 0x80000000u);
  return k + (negz ? 1u : 0u);  // ~0x80000000 + 1 = key of +0
}

// 1 / x in fp64: hardware estimate and one Newton step (a few ulps).
__device__ __forceinline__ double rcp_nr(double x) {
  const double r = __builtin_amdgcn_rcp(x);
  return __builtin_fma(r, __builtin_fma(-x, r, 1.0), r);
}

// FULL: every bucket of the launch holds D values (the last, shorter bucket
// has a launch of its own, so the main grid carries no bounds tests).
// The second bound is the minimum number of waves per SIMD: 3 for the
// 256-thread instances, 4 (128 VGPRs) where keys live partly in LDS; none
// for the one-block launch of a short last bucket (no occupancy to keep,
// so no spilling to fit it).
template <int D, bool EF, bool FULL>
__global__ __launch_bounds__(D / elems_per_thread(D),
                             !FULL ? 1
                             : D / elems_per_thread(D) == 256 ? 3
                             : (keys_in_regs(D) < elems_per_thread(D) ? 4 : 1))
void k_binopt_block(
    int64_t n, const float* __restrict__ g, float* __restrict__ e,
    uint8_t* __restrict__ codes, float* __restrict__ meta, int64_t code_bytes,
    int64_t first_bucket) {
  constexpr int E = elems_per_thread(D);
  constexpr int T = D / E;
  constexpr int NQ = E / 4;
  constexpr int NW = T / 64;
  constexpr int ER = keys_in_regs(D);  // keys 0 .. ER-1 in registers
  constexpr int EL = E - ER;           // keys ER .. E-1 in LDS
  struct Shared {
    // per bin, one column per lane: count << 48 plus the biased fixed-point sum
    unsigned long long h[kBins * kRow];
    float v[NW][2 * kCap];     // survivors, gathered per wave (the upper
                               // half takes the other lanes' stores)
    int wc[NW];                // survivors per wave
    double rd[4][NW];          // per-wave partials: S, sums below the ranges
    uint32_t ru[2][NW];        // per-wave key minima / maxima
    uint32_t kthr;             // exact stage result: threshold key,
    float la, lb;              //   levels,
    int flag;                  //   0 done, 1 recompute sums, 2 fall back
    double ks;                 //   split position
    double s2[4][NW];          // compensated cluster sums (rare path)
    // the next level's ranges, from the first wave
    uint32_t nlo[2], nhi[2];
    int nk[2], nc[2], nst, nnr;
    long long nq[2];
    double nlb;
    // key ER + j of thread t at [j][t] (last: h keeps its 16-byte alignment)
    uint32_t kx[EL > 0 ? EL : 1][EL > 0 ? T : 1];
  };
  __shared__ __align__(16) Shared sh;

  const int tid = threadIdx.x, wv = tid >> 6, wl = tid & 63;
  const int b = wl;  // the bin of this lane in the bin stages (first wave)
  const int64_t bucket = first_bucket + blockIdx.x;
  const int64_t base = bucket * D;
  const int nj = FULL ? D : (int)((n - base) < D ? (n - base) : D);
  // whether held value m is in the gradient (recomputed at each use: kept,
  // the tests of the last bucket took one scalar register pair per value)
  const int rem = nj - 4 * tid;
  auto valid = [&](int m) {
    if constexpr (FULL) return true;
    else return 4 * T * (m / 4) + (m % 4) < (int)opaque((uint32_t)rem);
  };

  // ---- load p = g (+ e); thread t holds the float4s t, t + T, ...; keep
  //      the keys of the canonical values (-0 -> +0); whether the wave saw a
  //      -0 at all (one scalar mask: the residual of a -0 differs from that
  //      of +0 only when its level is +0, and that rare case re-reads p);
  //      bucket statistics on the way: key range and S = sum (fp64) -------
  uint32_t kk[ER];
  // held key m (m a compile-time index after unrolling)
  auto key = [&](int m) -> uint32_t {
    if (m < ER) return kk[m < ER ? m : 0];
    return sh.kx[m < ER ? 0 : m - ER][tid];
  };
  uint64_t zmask = 0ull;
  uint32_t kmn = 0xffffffffu, kmx = 0u;
  double S = 0.0;
  auto take = [&](int q, float4 x) {
    const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float v = xs[c];
      const uint32_t bits = __float_as_uint(v);
      const bool nz = bits == 0x80000000u;
      zmask |= __ballot(nz);
      const uint32_t kv = canon_key(bits, nz);
      if (4 * q + c < ER) kk[4 * q + c < ER ? 4 * q + c : 0] = kv;
      else sh.kx[4 * q + c < ER ? 0 : 4 * q + c - ER][tid] = kv;
      const bool ok = valid(4 * q + c);
      kmn = (ok & (kv < kmn)) ? kv : kmn;
      kmx = (ok & (kv > kmx)) ? kv : kmx;
      S = ok ? S + (double)v : S;
    }
  };
  if constexpr (FULL) {
    // at most eight float4s per stream in flight
    constexpr int QC = NQ < 8 ? NQ : 8;
#pragma unroll
    for (int q0 = 0; q0 < NQ; q0 += QC) {
      float4 xq[QC];
#pragma unroll
      for (int q = 0; q < QC; ++q) xq[q] = load4_nt(g + base + 4 * (tid + (int64_t)T * (q0 + q)));
      if constexpr (EF) {
#pragma unroll
        for (int q = 0; q < QC; ++q) {
          const float4 r = load4_nt(e + base + 4 * (tid + (int64_t)T * (q0 + q)));
          xq[q].x = xq[q].x + r.x;
          xq[q].y = xq[q].y + r.y;
          xq[q].z = xq[q].z + r.z;
          xq[q].w = xq[q].w + r.w;
        }
      }
#pragma unroll
      for (int q = 0; q < QC; ++q) take(q0 + q, xq[q]);
    }
  } else {
    // the last bucket: element-wise bounds, one float4 at a time
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      asm volatile("" ::: "memory");
      const int64_t i = base + 4 * (tid + (int64_t)T * q);
      float4 x = load4(g, i, n);
      if constexpr (EF) {
        const float4 r = load4(e, i, n);
        x.x = x.x + r.x;
        x.y = x.y + r.y;
        x.z = x.z + r.z;
        x.w = x.w + r.w;
      }
      take(q, x);
    }
  }

  kmn = group_min_u<64>(kmn);
  kmx = group_max_u<64>(kmx);
  S = group_sum_d<64>(S);
  if (wl == 0) {
    sh.ru[0][wv] = kmn;
    sh.ru[1][wv] = kmx;
    sh.rd[0][wv] = S;
  }
  __syncthreads();
  kmn = sh.ru[0][0];
  kmx = sh.ru[1][0];
  S = sh.rd[0][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    kmn = sh.ru[0][w] < kmn ? sh.ru[0][w] : kmn;
    kmx = sh.ru[1][w] > kmx ? sh.ru[1][w] : kmx;
    S = S + sh.rd[0][w];
  }
  // combined here, not where first used (the wave partials' loads were
  // otherwise kept in registers, or spilled, until the exact stage)
  asm volatile("" : "+v"(S));
  const double dn = (double)nj;

  // The histogram sums are fixed point: value x adds q = trunc(x 2^f), with
  // 2^f chosen so that |q| < 2^30 for every value; the LDS word holds
  // 2^48 + q + 2^30 (count from bit 48, a nonnegative sum below it: at most
  // 2^15 values of less than 2^31 stay below 2^46).  The sum of the
  // quantized values below any split is then exact, and |P_q - P| < nj 2^-f
  // =: dP.  F moves by at most 2 |a - b| d + 4 d^2 when P moves by d, and
  // |a - b| <= max - min.
  const float amax = fmaxf(fabsf(funkey(kmn)), fabsf(funkey(kmx)));
  int ex = 0;
  frexpf(amax, &ex);  // amax < 2^ex
  const int fsh = 30 - ex;
  const float fscale = ldexpf(1.0f, fsh);
  const double funit = ldexp(1.0, -fsh);  // value of one fixed-point unit
  const double dP = dn * funit;
  const double span = (double)funkey(kmx) - (double)funkey(kmn);
  const double errF = 2.0 * span * dP + 4.0 * dP * dP;

  // candidate ranges (keys, inclusive), the split position K and the
  // fixed-point sum below each range start, and the count in each (the same
  // in every thread)
  int nr = 1;
  uint32_t rlo0 = kmn, rhi0 = kmx, rlo1 = 0u, rhi1 = 0u;
  int rk0 = 0, rk1 = 0, rc0 = nj, rc1 = 0;
  long long rq0 = 0, rq1 = 0;
  double LB = -1.0;

  const bool split_exists = kmn < kmx;
  // 0: refining, 1: exact stage, 2: fall back to the sort.  Buckets whose
  // scale 2^f would leave fp32's range go to the sort directly.
  const bool sane = amax < 0x1p90f && amax > 0x1p-90f;
  int state = !split_exists ? 1 : (nj <= kCap ? 1 : (sane ? 0 : 2));
  // this lane's histogram column as an LDS-space pointer (32-bit address
  // arithmetic per insertion)
  typedef __attribute__((address_space(3))) unsigned long long lds_u64;
  lds_u64* const col = (lds_u64*)(sh.h + (wl & (kCols - 1)));
  auto hist_add = [&](int bin, uint32_t k) {
    const uint32_t q = (uint32_t)((int)(kval(k) * fscale) + (1 << 30));
    const unsigned long long v = (0x10000ull << 32) | q;
    __atomic_fetch_add(col + __umul24((uint32_t)bin, (uint32_t)kRow), v, __ATOMIC_RELAXED);
  };
  auto uni = [](uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); };
  auto uni64 = [](long long x) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
    return (long long)(((uint64_t)hi << 32) | lo);
  };

  for (int lev = 0; lev < kLevels && state == 0; ++lev) {
    const int cnt_prev = rc0 + rc1;
    const int lgb = nr == 2 ? 5 : 6;  // log2 of the bins per range
    const int nbr = 1 << lgb;
    // shift of each range: (hi - lo) >> sh < nbr
    const uint32_t span0 = rhi0 - rlo0, span1 = rhi1 - rlo1;
    const int sh0 = (span0 >> lgb) == 0u ? 0 : 32 - __clz((int)(span0 >> lgb));
    const int sh1 = (span1 >> lgb) == 0u ? 0 : 32 - __clz((int)(span1 >> lgb));
    // clear the histogram's columns (after every wave read the previous
    // level's), 16 bytes per store
    {
      ulonglong2* const h2 = reinterpret_cast<ulonglong2*>(sh.h);
#pragma unroll
      for (int i = tid; i < kBins * kCols / 2; i += T)
        h2[(i / (kCols / 2)) * (kRow / 2) + (i % (kCols / 2))] = make_ulonglong2(0ull, 0ull);
    }
    __syncthreads();
    if (lev == 0) {
      // one range, [min, max]: every value has a bin
#pragma unroll
      for (int m = 0; m < E; ++m) {
        if (!valid(m)) continue;
        const uint32_t k = key(m);
        hist_add((int)((k - rlo0) >> sh0), k);
      }
    } else if (nr == 1) {
#pragma unroll
      for (int m = 0; m < E; ++m) {
        const uint32_t k = key(m);
        const uint32_t t0 = k - rlo0;
        if (!valid(m) | (t0 > span0)) continue;
        hist_add((int)(t0 >> sh0), k);
      }
    } else {
#pragma unroll
      for (int m = 0; m < E; ++m) {
        const uint32_t k = key(m);
        const uint32_t t0 = k - rlo0, t1 = k - rlo1;
        const bool in0 = t0 <= span0;
        if (!valid(m) | !(in0 | (t1 <= span1))) continue;
        hist_add(in0 ? (int)(t0 >> sh0) : nbr + (int)(t1 >> sh1), k);
      }
    }
    __syncthreads();
    if (wv == 0) {
    // ---- per-bin totals (lane b holds bin b) -----------------------------
    long long bq = 0;
    int bc = 0;
    {
      const ulonglong2* h2 = reinterpret_cast<const ulonglong2*>(sh.h + b * kRow);
      unsigned long long tot = 0ull;
#pragma unroll
      for (int t = 0; t < kCols / 2; ++t) {
        const ulonglong2 v = h2[t];
        tot += v.x + v.y;
      }
      bc = (int)(tot >> 48);
      bq = (long long)(tot & 0xffffffffffffull) - ((long long)bc << 30);
    }
    // ---- edges: K and P at the bin's first edge --------------------------
    const int r = b >> lgb;     // range of this bin
    const int j = b - (r << lgb);  // bin within the range
    // prefix over the wave, the second range's restarted at its first bin
    const int inK = wave_inclusive(bc);
    const long long inQ = wave_inclusive(bq);
    const int cutK = r == 1 ? __builtin_amdgcn_readlane(inK, nbr - 1) : 0;
    const long long cutQ = r == 1 ? readlane64(inQ, nbr - 1) : 0ll;
    const int exK = inK - bc - cutK;
    const long long exQ = inQ - bq - cutQ;
    const uint32_t rlo = r == 0 ? rlo0 : rlo1, rhi = r == 0 ? rhi0 : rhi1;
    const int shr = r == 0 ? sh0 : sh1;
    const int Kb = (r == 0 ? rk0 : rk1) + exK;
    const long long Qb = (r == 0 ? rq0 : rq1) + exQ;
    const double Pb = (double)Qb * funit;
    const double bs = (double)bq * funit;
    const uint64_t klo64 = (uint64_t)rlo + ((uint64_t)j << shr);
    uint64_t khi64 = klo64 + ((uint64_t)1 << shr) - 1;
    if (khi64 > rhi) khi64 = rhi;
    const bool live = klo64 <= (uint64_t)rhi && bc > 0;
    const uint32_t klo = (uint32_t)(live ? klo64 : rlo);
    const uint32_t khi = (uint32_t)(live ? khi64 : rlo);
    // The splits inside the bin: (Kb + j, P) with j in [j0, j1] (the
    // bucket's ends excluded) and P - Pb between the lower boundary
    // max(j lo, bs - (c - j) hi) and the upper min(j hi, bs - (c - j) lo).
    // F is convex, so its maximum there is at a vertex: the bin's edges (or,
    // at a bucket end, the two boundary points at j0 or j1) and the two
    // corners of the boundaries.  F at an inner edge is also a lower bound.
    const double lo = (double)funkey(klo), hi = (double)funkey(khi);
    const double c = (double)bc;
    const bool ext0 = Kb == 0, ext1 = Kb + bc == nj;
    const double j0 = ext0 ? 1.0 : 0.0;
    const double j1 = ext1 ? c - 1.0 : c;
    const bool has = live && j0 <= j1;
    const double dK = (double)Kb;
    auto Lw = [&](double jj) { return Pb + fmax(jj * lo, bs - (c - jj) * hi); };
    auto Up = [&](double jj) { return Pb + fmin(jj * hi, bs - (c - jj) * lo); };
    double lb = -1.0, ub = -1.0;
    if (has) {
      const double fa = obj_fast(ext0 ? Lw(j0) : Pb, dK + j0, S, dn);
      const double fc = obj_fast(ext1 ? Up(j1) : Pb + bs, dK + j1, S, dn);
      ub = fmax(fa, fc);
      lb = fmax(ext0 ? -1.0 : fa, ext1 ? -1.0 : fc);
      if (hi > lo) {
        const double rd = rcp_nr(hi - lo);
        const double jl = (c * hi - bs) * rd;  // lower boundary's corner
        const double ju = (bs - c * lo) * rd;  // upper boundary's corner
        if (jl > j0 && jl < j1) ub = fmax(ub, obj_fast(Pb + jl * lo, dK + jl, S, dn));
        if (ju > j0 && ju < j1) ub = fmax(ub, obj_fast(Pb + ju * hi, dK + ju, S, dn));
      }
    }
    // the other boundary point at a clipped end (bins holding the bucket's
    // smallest or largest value)
    if (__ballot(has & (ext0 | ext1)) != 0ull) {
      if (has & (ext0 | ext1)) {
        ub = fmax(ub, obj_fast(ext0 ? Up(j0) : Pb, dK + j0, S, dn));
        ub = fmax(ub, obj_fast(ext1 ? Lw(j1) : Pb + bs, dK + j1, S, dn));
      }
    }
    LB = fmax(LB, group_max_d<64>(lb));
    const double slack = 1e-12 * fabs(LB);
    const bool keep = live && ub + errF + slack >= LB - errF - slack;
    // ---- survivors -> at most two ranges ---------------------------------
    const uint64_t mask = (uint64_t)__ballot(keep);
    if (mask == 0ull) {
      state = 2;
    } else {
      const uint64_t m0 = nbr == 64 ? mask : mask & ((1ull << nbr) - 1ull);
      const uint64_t m1 = nr == 2 ? mask >> nbr : 0ull;
      int a0, a1, b0, b1;
      if (m0 != 0ull && m1 != 0ull) {
        a0 = __builtin_ctzll(m0);
        a1 = 63 - __builtin_clzll(m0);
        b0 = nbr + __builtin_ctzll(m1);
        b1 = nbr + 63 - __builtin_clzll(m1);
      } else {
        a0 = __builtin_ctzll(mask);
        const uint64_t run = ~(mask >> a0);  // first zero after the run
        a1 = run == 0ull ? 63 : a0 + __builtin_ctzll(run) - 1;
        const uint64_t rest = a1 == 63 ? 0ull : mask >> (a1 + 1);
        b0 = rest ? a1 + 1 + __builtin_ctzll(rest) : -1;
        b1 = 63 - __builtin_clzll(mask);
      }
      auto bin_lo = [&](int bn) {
        const int rr = bn >> lgb;
        return (rr == 0 ? rlo0 : rlo1) + (uint32_t)((uint64_t)(bn - (rr << lgb)) << (rr == 0 ? sh0 : sh1));
      };
      auto bin_hi = [&](int bn) {
        const int rr = bn >> lgb;
        const uint64_t h = (uint64_t)(rr == 0 ? rlo0 : rlo1) +
                           ((uint64_t)(bn - (rr << lgb) + 1) << (rr == 0 ? sh0 : sh1)) - 1;
        const uint32_t top = rr == 0 ? rhi0 : rhi1;
        return h > top ? top : (uint32_t)h;
      };
      // K at the chosen first and last edges and P at the first edges, from
      // the lanes of those bins (uniform indices)
      const int endK = Kb + bc;
      const int nk0 = __builtin_amdgcn_readlane(Kb, a0);
      const int nc0 = __builtin_amdgcn_readlane(endK, a1) - nk0;
      const long long qA = readlane64(Qb, a0);
      int nk1 = 0, nc1 = 0;
      long long nq1 = 0;
      const bool two = b0 >= 0;
      if (two) {
        nk1 = __builtin_amdgcn_readlane(Kb, b0);
        nc1 = __builtin_amdgcn_readlane(endK, b1) - nk1;
        nq1 = readlane64(Qb, b0);
      }
      const uint32_t nlo0 = bin_lo(a0), nhi0 = bin_hi(a1);
      const uint32_t nlo1 = two ? bin_lo(b0) : 0u, nhi1 = two ? bin_hi(b1) : 0u;
      rlo0 = nlo0;
      rhi0 = nhi0;
      rk0 = nk0;
      rq0 = qA;
      rc0 = nc0;
      nr = two ? 2 : 1;
      rlo1 = nlo1;
      rhi1 = nhi1;
      rk1 = nk1;
      rq1 = nq1;
      rc1 = nc1;
      // Large buckets stop refining once a level has not halved the
      // candidates: the rest are near-equal splits the bounds cannot part.
      if (rc0 + rc1 <= kCap) state = 1;
      else if (D >= 16384 && rc0 + rc1 <= kCapW && 2 * (rc0 + rc1) > cnt_prev) state = 3;
      else if (lev + 1 == kLevels) state = rc0 + rc1 <= kCapW ? 3 : 2;
    }
    if (wl == 0) {
      sh.nlo[0] = rlo0;
      sh.nhi[0] = rhi0;
      sh.nk[0] = rk0;
      sh.nq[0] = rq0;
      sh.nc[0] = rc0;
      sh.nlo[1] = rlo1;
      sh.nhi[1] = rhi1;
      sh.nk[1] = rk1;
      sh.nq[1] = rq1;
      sh.nc[1] = rc1;
      sh.nnr = nr;
      sh.nst = state;
      sh.nlb = LB;
    }
    }  // first wave
    __syncthreads();
    // the same in every lane: scalar registers from here
    rlo0 = uni(sh.nlo[0]);
    rhi0 = uni(sh.nhi[0]);
    rk0 = (int)uni((uint32_t)sh.nk[0]);
    rq0 = uni64(sh.nq[0]);
    rc0 = (int)uni((uint32_t)sh.nc[0]);
    rlo1 = uni(sh.nlo[1]);
    rhi1 = uni(sh.nhi[1]);
    rk1 = (int)uni((uint32_t)sh.nk[1]);
    rq1 = uni64(sh.nq[1]);
    rc1 = (int)uni((uint32_t)sh.nc[1]);
    nr = (int)uni((uint32_t)sh.nnr);
    state = (int)uni((uint32_t)sh.nst);
    LB = __longlong_as_double(uni64(__double_as_longlong(sh.nlb)));
    __syncthreads();  // the next level clears the histogram
  }
  if (state == 0) state = 2;

  if (state == 2) {
    // not resolved: NaN levels mark the bucket for the sort-based kernel;
    // codes and residual are left to it
    if (tid == 0) {
      meta[2 * bucket + 0] = __builtin_nanf("");
      meta[2 * bucket + 1] = __builtin_nanf("");
    }
    return;
  }

  // ---- exact stage over the values of the ranges --------------------------
  float la, lb_;
  uint32_t kthr;
  if (!split_exists) {
    la = lb_ = funkey(kmn);
    kthr = 0xffffffffu;  // every code 0 (keys of finite values are below
                         // 0xff800000)
  } else {
    if (state == 3) {
      // The levels ran out, or at d >= 16384 stopped halving, with
      // kCap < survivors <= kCapW (the bounds' slack for the fixed-point
      // sums keeps near-maximal splits of flat objectives alive): the same
      // exact stage with four survivors per lane.  One pass:
      // the fp64 sums below each range start, and the survivors appended to
      // one list in the histogram's LDS (no longer needed), at offsets from a
      // per-wave reservation.
      float* const list = reinterpret_cast<float*>(sh.h);
      if (tid == 0) sh.wc[0] = 0;
      __syncthreads();
      double p0 = 0.0, p1 = 0.0;
#pragma unroll
      for (int m = 0; m < E; ++m) {
        const bool v = valid(m);
        const uint32_t k = key(m);
        const float x = kval(k);
        p0 = (v & (k < rlo0)) ? p0 + (double)x : p0;
        p1 = (v & (k < rlo1)) ? p1 + (double)x : p1;
        const bool in = v & ((k - rlo0 <= rhi0 - rlo0) | (k - rlo1 <= rhi1 - rlo1));
        const uint64_t bal = (uint64_t)__ballot(in);
        if (bal != 0ull) {
          int wbase = 0;
          if (wl == 0) wbase = atomicAdd(&sh.wc[0], __popcll(bal));
          wbase = __shfl(wbase, 0, 64);
          const int pos = wbase + (int)__builtin_amdgcn_mbcnt_hi(
                                      (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
          if (in && pos < kCapW) list[pos] = x;
        }
      }
      p0 = group_sum_d<64>(p0);
      p1 = group_sum_d<64>(p1);
      if (wl == 0) {
        sh.rd[2][wv] = p0;
        sh.rd[3][wv] = p1;
      }
      __syncthreads();
      p0 = sh.rd[2][0];
      p1 = sh.rd[3][0];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        p0 = p0 + sh.rd[2][w];
        p1 = p1 + sh.rd[3][w];
      }
      if (wv == 0) {
        const int cnt = sh.wc[0];
        // positions 4 wl .. 4 wl + 3 of the sorted survivors
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pos = 4 * wl + r;
          y[r] = pos < cnt && pos < kCapW ? list[pos] : __builtin_inff();
        }
        sv_levels<4, kCapW, 2>(y, wl);
        double own[4], tl = 0.0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          own[r] = 4 * wl + r < cnt ? (double)y[r] : 0.0;
          tl = tl + own[r];
        }
        const double lane_pre = group_inclusive<64>(tl) - tl;  // sum before the lane
        double pre[4];
        {
          double acc = lane_pre;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pre[r] = acc;  // sum before position 4 wl + r
            acc = acc + own[r];
          }
        }
        const int off1 = rc0;  // start of range 1
        double pre_off1 = 0.0;
        if (off1 < cnt) {
          const int ro = off1 & 3;
          const double mine = ro == 0 ? pre[0] : ro == 1 ? pre[1] : ro == 2 ? pre[2] : pre[3];
          pre_off1 = __longlong_as_double(readlane64(__double_as_longlong(mine), off1 >> 2));
        }
        const float y_prev_lane = __shfl_up(y[3], 1, 64);
        double bestF = -1.0;
        int bestK = 0x7fffffff;
        uint32_t bestT = 0u;
        double bestP = 0.0;
        auto consider = [&](int k, double P, uint32_t kt) {
          if (k <= 0 || k >= nj) return;
          const double f = obj_fast(P, (double)k, S, dn);
          if (f > bestF || (f == bestF && k < bestK)) {
            bestF = f;
            bestK = k;
            bestT = kt;
            bestP = P;
          }
        };
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pos = 4 * wl + r;
          if (pos < cnt) {
            const bool r1 = pos >= off1;
            const int start = r1 ? off1 : 0;
            const float yp = r == 0 ? y_prev_lane : y[r > 0 ? r - 1 : 0];
            const bool distinct = pos == start || yp < y[r];
            const int k = (r1 ? rk1 : rk0) + (pos - start);
            const double P = (r1 ? p1 : p0) + (pre[r] - (r1 ? pre_off1 : 0.0));
            if (distinct) consider(k, P, fkey(y[r]));
            if (pos + 1 == (r1 ? cnt : off1)) {  // after the range's last value
              const int k2 = r1 ? rk1 + rc1 : rk0 + rc0;
              const double P2 = (r1 ? p1 : p0) + ((pre[r] + own[r]) - (r1 ? pre_off1 : 0.0));
              consider(k2, P2, (r1 ? rhi1 : rhi0) + 1u);
            }
          }
        }
        // lanes hold increasing splits: the first lane reaching the maximum
        const double gF = group_max_d<64>(bestF);
        const uint64_t at_max = (uint64_t)__ballot(bestF == gF);
        const int win = __builtin_ctzll(at_max);
        const int gK = __builtin_amdgcn_readlane(bestK, win);
        const uint32_t kt = (uint32_t)__builtin_amdgcn_readlane((int)bestT, win);
        const double Ps = __longlong_as_double(readlane64(__double_as_longlong(bestP), win));
        if (wl == 0) {
          if (gF < 0.0 || cnt > kCapW || cnt != rc0 + rc1) {
            sh.flag = 2;
          } else {
            const double ks = (double)gK;
            sh.kthr = kt;
            sh.ks = ks;
            sh.la = (float)(Ps / ks);
            sh.lb = (float)((S - Ps) / (dn - ks));
            const double tiny = 0x1p-20 * (double)amax * dn;
            sh.flag = (fabs(Ps) < tiny || fabs(S - Ps) < tiny) ? 1 : 0;
          }
        }
      }
    } else {
      // one pass: the fp64 sums below each range start, and the survivors
      // appended to this wave's list (offsets from the wave's ballot); with
      // one range (nr is the same in every thread) the second range's sum and
      // test are left out (p1 stays 0, no value lies in it)
      double p0 = 0.0, p1 = 0.0;
      int woff = 0;
      // x times 1.0 or 0.0 (the selected constant has a zero low word)
      auto gate = [](bool c) { return __hiloint2double(c ? 0x3ff00000 : 0, 0); };
      auto pass = [&](auto two_tag) {
        constexpr bool TWO = decltype(two_tag)::value;
  #pragma unroll
        for (int m = 0; m < E; ++m) {
          const bool v = valid(m);
          const uint32_t k = key(m);
          const float x = kval(k);
          const double dx = (double)x;
          p0 = __builtin_fma(dx, gate(v & (k < rlo0)), p0);
          if constexpr (TWO) p1 = __builtin_fma(dx, gate(v & (k < rlo1)), p1);
          const bool in0 = v & (k - rlo0 <= rhi0 - rlo0);
          const bool in1 = TWO && (v & (k - rlo1 <= rhi1 - rlo1));
          const uint64_t bal = TWO ? ((uint64_t)__ballot(in0) | (uint64_t)__ballot(in1))
                                   : (uint64_t)__ballot(in0);
          // most slots hold no survivor in any lane of the wave: the gather is
          // skipped for them (a wave-uniform branch)
          if (bal != 0ull) {
            const int pos = woff + (int)__builtin_amdgcn_mbcnt_hi(
                                       (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            // every lane stores (no branch per value): the others to a slot
            // of their own above the list
            sh.v[wv][((in0 | in1) & (pos < kCap)) ? pos : kCap + wl] = x;
            woff += __popcll(bal);
          }
        }
      };
      if (nr == 2) pass(std::true_type{});
      else pass(std::false_type{});
      p0 = group_sum_d<64>(p0);
      p1 = group_sum_d<64>(p1);
      if (wl == 0) {
        sh.rd[2][wv] = p0;
        sh.rd[3][wv] = p1;
        sh.wc[wv] = woff;
      }
      __syncthreads();
      p0 = sh.rd[2][0];
      p1 = sh.rd[3][0];
  #pragma unroll
      for (int w = 1; w < NW; ++w) {
        p0 = p0 + sh.rd[2][w];
        p1 = p1 + sh.rd[3][w];
      }
      if (wv == 0) {
        // one survivor per lane (the waves' lists in wave order), sorted
        int cnt = 0;
        float y[1] = {__builtin_inff()};
  #pragma unroll
        for (int w = 0; w < NW; ++w) {
          const int cw = sh.wc[w];
          const int at = wl - cnt;
          if (at >= 0 && at < cw && at < kCap) y[0] = sh.v[w][at];
          cnt += cw;
        }
        sv_levels<1, kCap, 2>(y, wl);
        const double own = wl < cnt ? (double)y[0] : 0.0;
        const double pre0 = group_inclusive<64>(own) - own;  // sum before this position
        const int off1 = rc0;                                  // start of range 1
        const double pre_off1 = off1 < 64 ? __longlong_as_double(readlane64(__double_as_longlong(pre0), off1)) : 0.0;
        const float y_prev = __shfl_up(y[0], 1, 64);
        double bestF = -1.0;
        int bestK = 0x7fffffff;
        uint32_t bestT = 0u;
        double bestP = 0.0;
        // F to a few ulps: buckets whose best two splits are closer than
        // that are ties, and either split is correct there
        auto consider = [&](int k, double P, uint32_t kt) {
          if (k <= 0 || k >= nj) return;
          const double f = obj_fast(P, (double)k, S, dn);
          if (f > bestF || (f == bestF && k < bestK)) {
            bestF = f;
            bestK = k;
            bestT = kt;
            bestP = P;
          }
        };
        if (wl < cnt) {
          const bool r1 = wl >= off1;
          const int start = r1 ? off1 : 0;
          const bool distinct = wl == start || y_prev < y[0];
          const int k = (r1 ? rk1 : rk0) + (wl - start);
          const double P = (r1 ? p1 : p0) + (pre0 - (r1 ? pre_off1 : 0.0));
          if (distinct) consider(k, P, fkey(y[0]));
          // the split after the range's last value
          const bool last = wl + 1 == (r1 ? cnt : off1);
          if (last) {
            const int k2 = r1 ? rk1 + rc1 : rk0 + rc0;
            const double P2 = (r1 ? p1 : p0) + ((pre0 + own) - (r1 ? pre_off1 : 0.0));
            consider(k2, P2, (r1 ? rhi1 : rhi0) + 1u);
          }
        }
        // the largest F, then the smallest split: lanes hold increasing
        // splits, so the first lane reaching the maximum
        const double gF = group_max_d<64>(bestF);
        const uint64_t at_max = (uint64_t)__ballot(bestF == gF);
        const int win = __builtin_ctzll(at_max);
        const int gK = __builtin_amdgcn_readlane(bestK, win);
        const uint32_t kt = (uint32_t)__builtin_amdgcn_readlane((int)bestT, win);
        const double Ps = __longlong_as_double(readlane64(__double_as_longlong(bestP), win));
        if (wl == 0) {
          if (gF < 0.0 || cnt > kCap) {
            sh.flag = 2;  // no candidate (cannot happen when the bounds hold)
          } else {
            const double ks = (double)gK;
            sh.kthr = kt;
            sh.ks = ks;
            sh.la = (float)(Ps / ks);
            sh.lb = (float)((S - Ps) / (dn - ks));
            // cluster sums with cancellation beyond the plain fp64 sums'
            // accuracy (rare; the bucket's scale is max |p| times n): recompute
            // both sides with compensated sums
            const double tiny = 0x1p-20 * (double)amax * dn;
            sh.flag = (fabs(Ps) < tiny || fabs(S - Ps) < tiny) ? 1 : 0;
          }
        }
      }
    }
    __syncthreads();
    const int flag = sh.flag;
    if (flag == 2) {
      if (tid == 0) {
        meta[2 * bucket + 0] = __builtin_nanf("");
        meta[2 * bucket + 1] = __builtin_nanf("");
      }
      return;
    }
    kthr = sh.kthr;
    la = sh.la;
    lb_ = sh.lb;
    if (flag == 1) {
      Sum2 lo{0.0, 0.0}, hi{0.0, 0.0};
#pragma unroll
      for (int m = 0; m < E; ++m) {
        if (!valid(m)) continue;
        const uint32_t k = key(m);
        const double x = (double)kval(k);
        if (k < kthr) two_sum_add(lo, x);
        else two_sum_add(hi, x);
      }
      lo = group_sum2<64>(lo);
      hi = group_sum2<64>(hi);
      if (wl == 0) {
        sh.s2[0][wv] = lo.s;
        sh.s2[1][wv] = lo.c;
        sh.s2[2][wv] = hi.s;
        sh.s2[3][wv] = hi.c;
      }
      __syncthreads();
      Sum2 L{sh.s2[0][0], sh.s2[1][0]}, H{sh.s2[2][0], sh.s2[3][0]};
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        L = two_sum_merge(L, Sum2{sh.s2[0][w], sh.s2[1][w]});
        H = two_sum_merge(H, Sum2{sh.s2[2][w], sh.s2[3][w]});
      }
      const double ks = sh.ks;
      la = (float)((L.s + L.c) / ks);
      lb_ = (float)((H.s + H.c) / (dn - ks));
    }
  }
  if (tid == 0) {
    meta[2 * bucket + 0] = la;
    meta[2 * bucket + 1] = lb_;
  }
  if (codes == nullptr) return;  // levels only

  // ---- codes, packing, residual (element order) ---------------------------
  // A -0 keeps its sign in the residual only against a +0 level; a wave
  // holding a -0 in a bucket with a zero level re-reads p for its residual.
  const bool reread = EF && zmask != 0ull && (la == 0.f || lb_ == 0.f);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int64_t i0 = base + 4 * (tid + (int64_t)T * q);
    uint32_t field = 0u;
    float r[4];
    float4 praw = make_float4(0.f, 0.f, 0.f, 0.f);
    if (reread) {
      praw = load4(g, i0, n);
      const float4 er = load4(e, i0, n);
      praw.x = praw.x + er.x;
      praw.y = praw.y + er.y;
      praw.z = praw.z + er.z;
      praw.w = praw.w + er.w;
    }
    const float pr[4] = {praw.x, praw.y, praw.z, praw.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int m = 4 * q + c;
      const uint32_t k = key(m);
      const uint32_t code = (valid(m) && k >= kthr) ? 1u : 0u;
      field |= code << c;
      const float pv = reread ? pr[c] : kval(k);
      r[c] = pv - (code ? lb_ : la);
    }
    store_chunk<1, 4>(codes, i0, wl, field, code_bytes);
    if (EF && i0 < n) {
      if constexpr (FULL) store4_nt(e + i0, make_float4(r[0], r[1], r[2], r[3]));
      else store4(e, i0, n, make_float4(r[0], r[1], r[2], r[3]));
    }
  }
}

template <int D, bool EF>
void launch_ef(int64_t n, const float* g, float* e, uint8_t* codes, float* meta,
               int64_t code_bytes, hipStream_t st) {
  const int64_t nfull = n / D;
  const dim3 block(D / elems_per_thread(D));
  if (nfull > 0)
    hipLaunchKernelGGL((k_binopt_block<D, EF, true>), dim3((uint32_t)nfull), block, 0, st,
                       n, g, e, codes, meta, code_bytes, (int64_t)0);
  if (n % D != 0)
    hipLaunchKernelGGL((k_binopt_block<D, EF, false>), dim3(1), block, 0, st,
                       n, g, e, codes, meta, code_bytes, nfull);
}

template <int D>
int launch_one(int64_t n, const float* g, float* e, uint8_t* codes, float* meta,
               int64_t code_bytes, hipStream_t st) {
  if (e != nullptr) launch_ef<D, true>(n, g, e, codes, meta, code_bytes, st);
  else launch_ef<D, false>(n, g, e, codes, meta, code_bytes, st);
  return (int)hipGetLastError();
}

}  // namespace

bool binopt_prune_supported(int d) { return d >= 1024 && d <= 32768; }

int launch_binopt_prune(int d, int64_t n, const float* g, float* e,
                        uint8_t* codes, float* meta, int64_t code_bytes,
                        hipStream_t st) {
  switch (d) {
    case 1024: return launch_one<1024>(n, g, e, codes, meta, code_bytes, st);
    case 2048: return launch_one<2048>(n, g, e, codes, meta, code_bytes, st);
    case 4096: return launch_one<4096>(n, g, e, codes, meta, code_bytes, st);
    case 8192: return launch_one<8192>(n, g, e, codes, meta, code_bytes, st);
    case 16384: return launch_one<16384>(n, g, e, codes, meta, code_bytes, st);
    case 32768: return launch_one<32768>(n, g, e, codes, meta, code_bytes, st);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace gq
