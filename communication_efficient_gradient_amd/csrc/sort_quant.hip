// sort_quant.hip — quantizers whose levels need the bucket sorted:
//   BIN_OPT  the two-level split that minimises squared error (BinGrad-b),
//   ORQ      greedy multi-level selection minimising the random-rounding
//            variance, with optional clipping, then random rounding.
// ("Optimal Gradient Quantization Condition" review, §Proposed method.)
//
// One workgroup per bucket, T threads, E = d/T elements per thread.
//   1. load p = g (+ e) in element order (thread t: elements t + T*m);
//   2. (ORQ + clip) clip to +-clip_sigma * RMS;
//   3. bitonic sort of the bucket in LDS (absent tail slots hold +inf);
//   4. thread t then owns the sorted run [t*E, t*E + E) and the block runs
//      fp64 (segmented) prefix / suffix scans over it:
//        BIN_OPT  F(k) = P_k^2/k + Q_k^2/(n-k) for every split between
//                 distinct values, block argmax (smallest k on equality);
//        ORQ      L-2 greedy steps; each evaluates, for every distinct
//                 interior value c of every interval (a, b),
//                 G(c) = (b-c) * sum_{a<y<=c}(y-a) + (c-a) * sum_{c<y<b}(b-y)
//                 from segmented scans (all terms >= 0: no cancellation),
//                 and inserts the block argmax (smallest c on equality);
//   5. back in element order: codes, packing, residual.
// The bucket is read from HBM once; everything after the load is on-chip.
#include <type_traits>

#include "common.hpp"

namespace gq {
namespace {

template <int D>
struct SortCfg {
  static constexpr int E = D <= 8192 ? 8 : D / 1024;  // values per thread
  static constexpr int T = D / E;                      // 128 .. 1024 threads
  static constexpr int NW = T / 64;
};

// ------------------------------------------------------ block primitives --
// Block max of a float (all threads get the result).
template <int T>
__device__ __forceinline__ float block_maxf(float v, float* red) {
  v = group_max<64>(v);
  if constexpr (T > 64) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int w = 1; w < T / 64; ++w) v = fmaxf(v, red[w]);
  }
  return v;
}

template <int T>
__device__ __forceinline__ Sum2 block_sum2(Sum2 v, double* red) {
  v = group_sum2<64>(v);
  if constexpr (T > 64) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) {
      red[2 * wave] = v.s;
      red[2 * wave + 1] = v.c;
    }
    __syncthreads();
    v = Sum2{red[0], red[1]};
#pragma unroll 1
    for (int w = 1; w < T / 64; ++w) v = two_sum_merge(v, Sum2{red[2 * w], red[2 * w + 1]});
  }
  return v;
}

// Block argmax of (value, key): larger value wins, equal values -> smaller
// key.  Returns the winning key (all threads).  Threads without a candidate
// pass value = -1 (all real values are >= 0).
template <int T>
__device__ __forceinline__ int block_argmax(double v, int key, double* redv,
                                            int* redk, double* best_out) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double v2 = xshfl(v, o);
    const int k2 = xshfl(key, o);
    if (v2 > v || (v2 == v && k2 < key)) {
      v = v2;
      key = k2;
    }
  }
  if constexpr (T > 64) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) {
      redv[wave] = v;
      redk[wave] = key;
    }
    __syncthreads();
    v = redv[0];
    key = redk[0];
#pragma unroll 1
    for (int w = 1; w < T / 64; ++w) {
      const double v2 = redv[w];
      const int k2 = redk[w];
      if (v2 > v || (v2 == v && k2 < key)) {
        v = v2;
        key = k2;
      }
    }
  }
  *best_out = v;
  return key;
}

// Number of entries below x in a row of 16 ascending floats (+inf padded)
// in LDS, for x not above the row's last finite entry: 0 .. 15.
__device__ __forceinline__ int lds_rank16(const float* row, float x) {
  int pos = row[7] < x ? 8 : 0;
  pos += row[pos + 3] < x ? 4 : 0;
  pos += row[pos + 1] < x ? 2 : 0;
  pos += row[pos] < x ? 1 : 0;
  return pos;
}

// Carry for a block-wide segmented scan over per-thread aggregates (f, s):
// f = the thread's run contains a segment boundary, s = the sum that flows
// on to the next thread.  Combining an earlier aggregate a with a later b
// gives (a.f | b.f, b.f ? b.s : a.s + b.s).  Returns, for each thread, the
// combination of all threads before it (REV = false) or after it
// (REV = true); identity (0, 0).
template <int T, bool REV>
__device__ __forceinline__ double block_seg_carry(bool f, double s,
                                                  double* red_s, int* red_f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int fi = f ? 1 : 0;
  // inclusive scan within the wave, in lane order (or reverse lane order)
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double s2 = REV ? __shfl_down(s, o, 64) : __shfl_up(s, o, 64);
    const int f2 = REV ? __shfl_down(fi, o, 64) : __shfl_up(fi, o, 64);
    const bool valid = REV ? (lane + o < 64) : (lane >= o);
    if (valid) {
      if (!fi) s = s2 + s;
      fi |= f2;
    }
  }
  // exclusive: the inclusive value of the neighbouring lane
  double ex_s = REV ? __shfl_down(s, 1, 64) : __shfl_up(s, 1, 64);
  int ex_f = REV ? __shfl_down(fi, 1, 64) : __shfl_up(fi, 1, 64);
  if (REV ? lane == 63 : lane == 0) {
    ex_s = 0.0;
    ex_f = 0;
  }
  if constexpr (T > 64) {
    constexpr int NW = T / 64;
    __syncthreads();
    if (REV ? lane == 0 : lane == 63) {
      red_s[wave] = s;
      red_f[wave] = fi;
    }
    __syncthreads();
    // carry from the waves before this one (in scan order)
    double cs = 0.0;
    if (!REV) {
      for (int w = 0; w < wave; ++w) {
        if (!red_f[w]) cs = cs + red_s[w]; else cs = red_s[w];
      }
    } else {
      for (int w = NW - 1; w > wave; --w) {
        if (!red_f[w]) cs = cs + red_s[w]; else cs = red_s[w];
      }
    }
    // combine wave carry (earlier) with the lane-exclusive value (later)
    if (!ex_f) ex_s = cs + ex_s;
  }
  return ex_s;
}

// Bitonic sort in "flip" form (every comparator ascending): merge level K
// first compares position i with i ^ (K-1) (the mirror image inside its
// K-block), then with i ^ J for J = K/4, ..., 1; the smaller value always
// goes to the lower position.  Values are held E per thread in blocked
// order (thread t: positions t*E .. t*E+E-1).  Partners in the same thread
// are register compare-exchanges; partners up to 63 lanes away come through
// lane exchanges (DPP, lane swaps); partners in another wave go through LDS
// (lds: the T*E values, two barriers per stage).  Everything is unrolled at
// compile time.

// stage with partner i ^ MASK; MASK = K-1 (mirror) or J (power of two)
// WIDE: the sort spans 64 lanes or more (a wave or a workgroup).
template <int E, int MASK, bool MIRROR, bool WIDE>
__device__ __forceinline__ void fb_stage(float (&y)[E], float* lds, int tid,
                                         int lane) {
  constexpr int TOP = MIRROR ? (MASK + 1) / 2 : MASK;  // bit deciding lower
  if constexpr (MASK < E) {
    // partners inside the thread
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const int r2 = r ^ MASK;
      if (r2 <= r) continue;
      const float a = y[r], b = y[r2];
      y[r] = fminf(a, b);
      y[r2] = fmaxf(a, b);
    }
  } else {
    // partner thread t ^ LM; register r pairs with r (power of two) or with
    // E-1-r (mirror)
    constexpr int LM = MASK / E;
    const bool lower = (tid & (TOP / E)) == 0;
    float o[E];
    if constexpr (LM < 64) {
      // through the LDS crossbar (no VALU work), except, in groups of at
      // most 32 lanes (fewer exchanges in flight per lane group), the
      // partners that one DPP move reaches
      constexpr bool dpp = LM == 1 || LM == 2 || LM == 3 || LM == 7 || LM == 8 || LM == 15;
#pragma unroll
      for (int r = 0; r < E; ++r) {
        if constexpr (dpp && !WIDE) o[r] = xshfl(y[MIRROR ? E - 1 - r : r], LM);
        else o[r] = lane_xor_ds<LM>(y[MIRROR ? E - 1 - r : r]);
      }
    } else {
      float4* l4 = reinterpret_cast<float4*>(lds);
#pragma unroll
      for (int r = 0; r < E; r += 4)
        l4[(tid * E + r) / 4] = make_float4(y[r], y[r + 1], y[r + 2], y[r + 3]);
      __syncthreads();
      const int pt = tid ^ LM;
#pragma unroll
      for (int r = 0; r < E; r += 4) {
        const float4 v = l4[(pt * E + r) / 4];
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (MIRROR) o[E - 1 - (r + c)] = vv[c];
          else o[r + c] = vv[c];
        }
      }
      __syncthreads();
    }
    (void)lane;
    // the smaller value to the lower thread: the median of (y, o, -inf) is
    // min(y, o), of (y, o, +inf) max(y, o); one instruction per value
    const float sel = lower ? -__builtin_inff() : __builtin_inff();
#pragma unroll
    for (int r = 0; r < E; ++r) y[r] = __builtin_amdgcn_fmed3f(y[r], o[r], sel);
  }
}

template <int E, int K, int J, bool WIDE>
__device__ __forceinline__ void fb_halves(float (&y)[E], float* lds, int tid,
                                          int lane) {
  if constexpr (J >= 1) {
    fb_stage<E, J, false, WIDE>(y, lds, tid, lane);
    fb_halves<E, K, J / 2, WIDE>(y, lds, tid, lane);
  }
}

template <int E, int N, int K>
__device__ __forceinline__ void fb_levels(float (&y)[E], float* lds, int tid,
                                          int lane) {
  constexpr bool WIDE = N / E >= 64;
  fb_stage<E, K - 1, true, WIDE>(y, lds, tid, lane);
  fb_halves<E, K, K / 4, WIDE>(y, lds, tid, lane);
  if constexpr (K < N) fb_levels<E, N, 2 * K>(y, lds, tid, lane);
}

// The 8 values of one thread ascending: a 19-comparator network (depth 6)
// in place of the bitonic levels 2, 4 and 8 (24 comparators).
__device__ __forceinline__ void sort8(float (&y)[8]) {
  constexpr int net[19][2] = {{0, 2}, {1, 3}, {4, 6}, {5, 7}, {0, 4}, {1, 5}, {2, 6},
                              {3, 7}, {0, 1}, {2, 3}, {4, 5}, {6, 7}, {2, 4}, {3, 5},
                              {1, 4}, {3, 6}, {1, 2}, {3, 4}, {5, 6}};
#pragma unroll
  for (int c = 0; c < 19; ++c) {
    const float a = y[net[c][0]], b = y[net[c][1]];
    y[net[c][0]] = fminf(a, b);
    y[net[c][1]] = fmaxf(a, b);
  }
}

// Sort N = T*E values (T threads of a workgroup, or the lanes of one group
// when N <= 64*E and lds is unused) ascending in blocked order.  `tid` is
// the thread's index among the N/E participants.
template <int E, int N>
__device__ __forceinline__ void flip_bitonic(float (&y)[E], float* lds,
                                             int tid) {
  if constexpr (E == 8 && N > 8) {
    sort8(y);
    fb_levels<E, N, 16>(y, lds, tid, tid & 63);
  } else {
    fb_levels<E, N, 2>(y, lds, tid, tid & 63);
  }
}

struct SortShared {
  double red_d[2 * 16];
  double red_v[16];
  int red_i[16];
  int red_k[16];
  float lev[16];
  float thr;
};

// One bucket by one workgroup (the body of k_sort_quant).
template <int SCHEME, int BITS, int D>
__device__ __forceinline__ void sort_quant_bucket(
    int64_t bucket, int64_t n, const float* __restrict__ g, float* __restrict__ e,
    uint32_t k0, uint32_t k1, uint32_t step, int L, int flags, float clip_sigma,
    uint8_t* __restrict__ codes, float* __restrict__ meta, int64_t code_bytes,
    uint32_t A4, int W) {
  constexpr int T = SortCfg<D>::T;
  constexpr int E = SortCfg<D>::E;
  __shared__ float sorted[D];
  __shared__ SortShared sh;

  const int tid = threadIdx.x;
  const int64_t base = bucket * D;
  const int nj = (int)((n - base) < D ? (n - base) : D);

  // ---- 1. load p = g (+ e); element order: thread t holds the float4s
  //         t, t + T, ... of the bucket -------------------------------------
  constexpr int NQ = E / 4;
  // For d <= 4096 p stays in registers for the coding pass, so the bucket is
  // read once, nontemporally.  Larger buckets read it again in the coding
  // pass: keeping it costs 10 VGPRs, which at 1024 threads per block leaves
  // room for one block per CU instead of two (BinGrad-b + EF on 1B, d = 8192:
  // 13.0 -> 17.6 ms), and at d = 32768 registers are at the limit already.
  constexpr bool KEEP = E <= 8 && T <= 512;
  float p[E];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int64_t i = base + 4 * (tid + (int64_t)T * q);
    const bool nt = KEEP && i + 4 <= n;
    float4 x = nt ? load4_nt(g + i) : load4(g, i, n);
    if (e != nullptr) {
      const float4 r = nt ? load4_nt(e + i) : load4(e, i, n);
      x.x = x.x + r.x;
      x.y = x.y + r.y;
      x.z = x.z + r.z;
      x.w = x.w + r.w;
    }
    p[4 * q + 0] = x.x;
    p[4 * q + 1] = x.y;
    p[4 * q + 2] = x.z;
    p[4 * q + 3] = x.w;
  }
  auto epos = [&](int m) { return 4 * (tid + T * (m / 4)) + (m % 4); };

  // ---- 2. clip (ORQ) -----------------------------------------------------
  const bool clip = (flags & GQ_FLAG_CLIP) != 0;
  float C = __builtin_inff();
  if (SCHEME == ORQ && clip) {
    Sum2 sq{0.0, 0.0};
#pragma unroll
    for (int m = 0; m < E; ++m)
      if (epos(m) < nj) two_sum_add(sq, (double)p[m] * (double)p[m]);
    sq = block_sum2<T>(sq, sh.red_d);
    const double sigma = sqrt((sq.s + sq.c) / (double)nj);
    C = (float)((double)clip_sigma * sigma);
  }
  // (C = +inf without clipping: the median of x, -C, C is then x)
  auto clipped = [&](float x) {
    if constexpr (SCHEME == ORQ) return __builtin_amdgcn_fmed3f(x, -C, C);
    else return x;
  };

  // ---- 3. sort (canonical +0, +inf padding), then publish it in LDS ------
  {
    float y[E];
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const float x = clipped(p[m]);
      y[m] = epos(m) < nj ? (x == 0.f ? 0.f : x) : __builtin_inff();
    }
    flip_bitonic<E, D>(y, sorted, tid);
    float4* l4 = reinterpret_cast<float4*>(sorted);
#pragma unroll
    for (int r = 0; r < E; r += 4)
      l4[(tid * E + r) / 4] = make_float4(y[r], y[r + 1], y[r + 2], y[r + 3]);
    __syncthreads();
  }

  // sorted run of this thread
  const int r0 = tid * E;
  const float y_next_run = (r0 + E < D) ? sorted[r0 + E] : __builtin_inff();
  const float y_prev_run = r0 > 0 ? sorted[r0 - 1] : -__builtin_inff();

  float lvl_a = 0.f, lvl_b = 0.f;  // BIN levels
  float thr = 0.f;
  bool no_split = false;

  if constexpr (SCHEME == BIN_OPT) {
    // ---- 4a. best split -------------------------------------------------
    double tot = 0.0;
#pragma unroll
    for (int m = 0; m < E; ++m)
      if (r0 + m < nj) tot = tot + (double)sorted[r0 + m];
    // prefix before this run, suffix after it (plain fp64 scans)
    const double pre = block_seg_carry<T, false>(false, tot, sh.red_d, sh.red_i);
    const double suf = block_seg_carry<T, true>(false, tot, sh.red_d, sh.red_i);
    double best = -1.0;
    int bestk = 0x7fffffff;
    // Q for each split: the suffix sum after each position of the run.
    double Qrun[E];
    {
      double acc = suf;
#pragma unroll
      for (int m = E - 1; m >= 0; --m) {
        Qrun[m] = acc;  // sum of positions > r0 + m
        if (r0 + m < nj) acc = acc + (double)sorted[r0 + m];
      }
    }
    double P = pre;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const int pos = r0 + m;
      if (pos < nj) P = P + (double)sorted[pos];
      const int k = pos + 1;  // split: positions < k below
      if (k < nj) {
        const float yk = (m + 1 < E) ? sorted[pos + 1] : y_next_run;
        if (sorted[pos] < yk) {
          const double F = P * P / (double)k + Qrun[m] * Qrun[m] / (double)(nj - k);
          if (F > best) {
            best = F;
            bestk = k;
          }
        }
      }
    }
    double bestF;
    const int kstar = block_argmax<T>(best, bestk, sh.red_v, sh.red_k, &bestF);
    if (bestF < 0.0) {
      no_split = true;
      thr = sorted[0];
      lvl_a = lvl_b = sorted[0];
    } else {
      thr = sorted[kstar];
      // levels: means of the two sides, near-exact fp64 sums
      Sum2 lo{0.0, 0.0}, hi{0.0, 0.0};
#pragma unroll
      for (int m = 0; m < E; ++m) {
        const int pos = r0 + m;
        if (pos < kstar) two_sum_add(lo, (double)sorted[pos]);
        else if (pos < nj) two_sum_add(hi, (double)sorted[pos]);
      }
      lo = block_sum2<T>(lo, sh.red_d);
      hi = block_sum2<T>(hi, sh.red_d);
      lvl_a = (float)((lo.s + lo.c) / (double)kstar);
      lvl_b = (float)((hi.s + hi.c) / (double)(nj - kstar));
    }
    if (tid == 0) {
      meta[2 * bucket + 0] = lvl_a;
      meta[2 * bucket + 1] = lvl_b;
    }
  } else {
    // ---- 4b. ORQ greedy levels -------------------------------------------
    const float ymin = sorted[0], ymax = sorted[nj - 1];
    if (tid == 0) {
      sh.lev[0] = ymin;
      sh.lev[1] = ymax;
    }
    int cnt = 2;
    if (ymin == ymax) {
      if (tid < L) sh.lev[tid] = ymin;
      cnt = L;
    }
    __syncthreads();
    while (cnt < L) {
      // segment of each sorted value: last level <= y
      float lv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) lv[j] = j < cnt ? sh.lev[j] : __builtin_inff();
      int seg[E];
      float a_of[E], b_of[E];
      bool head[E], tail[E];
      double va[E], vb[E];
      int seg_prev = -1;
      {
        // segment of the value just before this run
        int sp = -1;
        if (r0 > 0) {
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (lv[j] <= y_prev_run) sp = j;
        }
        seg_prev = sp;
      }
      int seg_next = -1;
      {
        int sn = -1;
        if (r0 + E < nj) {
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (lv[j] <= y_next_run) sn = j;
        }
        seg_next = sn;
      }
#pragma unroll
      for (int m = 0; m < E; ++m) {
        const float y = sorted[r0 + m];
        int sj = 0;
        float a = lv[0], b = lv[0];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (lv[j] <= y) {
            sj = j;
            a = lv[j];
            b = (j + 1 < 16 && j + 1 < cnt) ? lv[j + 1 < 16 ? j + 1 : 15] : lv[j];
          }
        }
        seg[m] = sj;
        a_of[m] = a;
        b_of[m] = b;
        const bool real = r0 + m < nj;
        va[m] = real ? (double)y - (double)a_of[m] : 0.0;
        vb[m] = real ? (double)b_of[m] - (double)y : 0.0;
      }
#pragma unroll
      for (int m = 0; m < E; ++m) {
        head[m] = (m == 0) ? (seg_prev != seg[0]) : (seg[m] != seg[m - 1]);
        tail[m] = (m == E - 1) ? (seg_next != seg[E - 1]) : (seg[m] != seg[m + 1]);
      }
      // forward aggregate for A (sum over the run's last segment piece)
      bool fa = false;
      double sa = 0.0;
#pragma unroll
      for (int m = 0; m < E; ++m) {
        if (head[m]) {
          fa = true;
          sa = va[m];
        } else {
          sa = sa + va[m];
        }
      }
      // reverse aggregate for B (sum over the run's first segment piece)
      bool fb = false;
      double sb = 0.0;
#pragma unroll
      for (int m = E - 1; m >= 0; --m) {
        if (tail[m]) {
          fb = true;
          sb = vb[m];
        } else {
          sb = sb + vb[m];
        }
      }
      const double ca = block_seg_carry<T, false>(fa, sa, sh.red_d, sh.red_i);
      const double cb = block_seg_carry<T, true>(fb, sb, sh.red_d, sh.red_i);
      // B: exclusive suffix within the segment
      double B[E];
      {
        double run = cb;
#pragma unroll
        for (int m = E - 1; m >= 0; --m) {
          if (tail[m]) {
            B[m] = 0.0;
            run = vb[m];
          } else {
            B[m] = run;
            run = run + vb[m];
          }
        }
      }
      double best = -1.0;
      int bestk = 0x7fffffff;
      {
        double A = ca;
#pragma unroll
        for (int m = 0; m < E; ++m) {
          A = head[m] ? va[m] : A + va[m];
          const int pos = r0 + m;
          const float y = sorted[pos];
          const float ynext = (m + 1 < E) ? sorted[pos + 1] : y_next_run;
          const bool cand = pos < nj && seg[m] + 1 < cnt && y > a_of[m] &&
                            (pos + 1 >= nj || ynext != y);
          if (cand) {
            const double c = (double)y;
            const double G = ((double)b_of[m] - c) * A + (c - (double)a_of[m]) * B[m];
            if (G > best) {
              best = G;
              bestk = pos;
            }
          }
        }
      }
      double bestG;
      const int kstar = block_argmax<T>(best, bestk, sh.red_v, sh.red_k, &bestG);
      __syncthreads();
      if (bestG < 0.0) {
        // fewer distinct values than levels: repeat the maximum
        if (tid == 0)
          for (int j = cnt; j < L; ++j) sh.lev[j] = ymax;
        cnt = L;
      } else {
        if (tid == 0) {
          const float c = sorted[kstar];
          int pos = cnt;
          while (pos > 0 && sh.lev[pos - 1] > c) {
            sh.lev[pos] = sh.lev[pos - 1];
            --pos;
          }
          sh.lev[pos] = c;
        }
        ++cnt;
      }
      __syncthreads();
    }
    if (tid < L) meta[bucket * L + tid] = sh.lev[tid];
    // +inf past the L levels, for the search of the coding pass
    if (tid >= L && tid < 16) sh.lev[tid] = __builtin_inff();
    __syncthreads();
  }

  if (codes == nullptr) return;  // levels only

  // ---- 5. codes, packing, residual (element order; p kept, or the bucket
  //         read again: the same g + e in fp32) -----------------------------
  const int lane = tid & 63;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int64_t i0 = base + 4 * (tid + (int64_t)T * q);
    float4 pv;
    if constexpr (KEEP) {
      pv = make_float4(p[4 * q + 0], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3]);
    } else {
      pv = load4(g, i0, n);
      if (e != nullptr) {
        const float4 r = load4(e, i0, n);
        pv.x = pv.x + r.x;
        pv.y = pv.y + r.y;
        pv.z = pv.z + r.z;
        pv.w = pv.w + r.w;
      }
    }
    const float px[4] = {pv.x, pv.y, pv.z, pv.w};
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (SCHEME == ORQ) {
      // random words, or (nearest) words whose u is exactly 1/2: the value
      // then rounds up iff q > 1/2
      w = make_uint4(kHalfWord, kHalfWord, kHalfWord, kHalfWord);
      if (!(flags & GQ_FLAG_NEAREST)) {
        const uint64_t ctr = (uint64_t)i0 >> 2;
        w = philox4x32_10(k0, k1, (uint32_t)ctr, (uint32_t)(ctr >> 32), step, 0u);
      }
    }
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    // BITS-bit codes, or (dense) 4-bit digits turned into one base-L
    // number at the store
    uint32_t field = 0u;
    float rr[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t code = 0u;
      float xh = 0.f;
      if constexpr (SCHEME == BIN_OPT) {
        code = (!no_split && px[c] >= thr) ? 1u : 0u;
        xh = code ? lvl_b : lvl_a;
      } else {
        // the levels around x by binary search in LDS: a value on a level
        // takes it (the first equal one), otherwise it rounds between the
        // levels below and above
        const float x = clipped(px[c]);
        const int above = lds_rank16(sh.lev, x);  // levels below x
        const float hi = sh.lev[above];
        const float lo = sh.lev[above > 0 ? above - 1 : 0];
        const float qf = (x - lo) / (hi - lo);
        const bool up = u24(ws[c]) < qf;
        const bool on = hi == x;
        code = (uint32_t)(on ? above : above - 1 + (up ? 1 : 0));
        xh = on ? x : (up ? hi : lo);
      }
      if (i0 + c >= n) code = 0u;
      field |= code << ((BITS == 0 ? 4 : BITS) * c);
      rr[c] = px[c] - xh;
    }
    if constexpr (BITS == 0)
      store_dense_chunk(codes, i0 - 4 * lane, nibbles_to_base(field, L), A4, W,
                        code_bytes);
    else
      store_chunk<BITS, 4>(codes, i0, lane, field, code_bytes);
    if (e != nullptr && i0 < n) {
      if (i0 + 4 <= n) store4_nt(e + i0, make_float4(rr[0], rr[1], rr[2], rr[3]));
      else store4(e, i0, n, make_float4(rr[0], rr[1], rr[2], rr[3]));
    }
  }
}

// A workgroup per bucket, or (redo) only the buckets the sort-free BinGrad-b
// kernel marked with NaN levels: then a workgroup checks 64 buckets (one
// level read per lane of its first wave) and sorts the marked ones in turn,
// so the pass costs a grid of nb / 64 short workgroups rather than nb (and
// marked buckets, which are rare, seldom share a workgroup).
template <int SCHEME, int BITS, int D>
__global__ __launch_bounds__(SortCfg<D>::T) void k_sort_quant(
    int64_t n, const float* __restrict__ g, float* __restrict__ e,
    uint32_t k0, uint32_t k1, uint32_t step, int L, int flags, float clip_sigma,
    uint8_t* __restrict__ codes, float* __restrict__ meta, int64_t code_bytes,
    uint32_t A4, int W, int redo) {
  if constexpr (SCHEME == BIN_OPT) {
    if (redo) {
      __shared__ uint64_t marks;
      const int64_t nb = (n + D - 1) / D;
      const int64_t first = (int64_t)blockIdx.x * 64;
      if (threadIdx.x < 64) {
        const int64_t b = first + threadIdx.x;
        const float lv = b < nb ? meta[2 * b] : 0.f;
        const uint64_t m = (uint64_t)__ballot(lv != lv);
        if (threadIdx.x == 0) marks = m;
      }
      __syncthreads();
      // the same in every thread: scalar, so the loop is workgroup-uniform
      const uint64_t mv = marks;
      uint64_t mw = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(mv >> 32)) << 32) |
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)mv);
      while (mw != 0ull) {
        const int bit = __builtin_ctzll(mw);
        mw &= mw - 1ull;
        sort_quant_bucket<SCHEME, BITS, D>(first + bit, n, g, e, k0, k1, step, L, flags,
                                           clip_sigma, codes, meta, code_bytes, A4, W);
        __syncthreads();  // the next bucket reuses the LDS
      }
      return;
    }
  }
  sort_quant_bucket<SCHEME, BITS, D>(blockIdx.x, n, g, e, k0, k1, step, L, flags,
                                     clip_sigma, codes, meta, code_bytes, A4, W);
}

// ------------------------------------------- one lane group per bucket --
// d <= 512: a group of G = d/8 lanes of one wavefront owns a bucket and keeps
// it in registers, E = 8 values per lane; a 256-thread workgroup holds 256/G
// buckets.  Element order (I/O): group lane t holds elements 4*(t + G*q) + c,
// q < 2, c < 4, so each 128-bit load of a group reads 4*G consecutive
// floats.  Sorted order: group lane t holds sorted positions 8t .. 8t+7.  The
// bitonic network runs in registers (partners in the same lane: compare-
// exchange; partners j/8 lanes away: DPP / lane swaps in the group), so the
// sort needs no LDS and no barrier.  The selection steps are those of the
// workgroup kernel above, with group-wide scans and argmax.
constexpr int kGroupThreads = 256;

// Values per lane and lanes per bucket.  8 values per lane keeps these
// kernels near 100-140 VGPRs; 16 per lane (fewer lanes per bucket, so
// cheaper scans and reductions) measured slower at half the occupancy.
template <int D>
struct WaveCfg {
  static constexpr int E = 8;
  static constexpr int G = D / E;
};

// DPP moves (no LDS): the value N lanes lower in the same 16-lane row (0 in
// the row's first N lanes), and the last lane of the previous row (BC = 15:
// rows 1 and 3) or lane 31 (BC = 31: rows 2 and 3), 0 elsewhere.
template <int N>
__device__ __forceinline__ int dpp_shr(int v) {
  // every lane written (bound_ctrl zero-fills the first N of a row), so no
  // old value to set up
  return __builtin_amdgcn_mov_dpp(v, 0x110 + N, 0xF, 0xF, true);
}
template <int BC>
__device__ __forceinline__ int dpp_bcast(int v) {
  return __builtin_amdgcn_update_dpp(0, v, BC == 15 ? 0x142 : 0x143,
                                     BC == 15 ? 0xA : 0xC, 0xF, false);
}
template <int N>
__device__ __forceinline__ double dpp_shr(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)dpp_shr<N>((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)dpp_shr<N>((int)(uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
template <int BC>
__device__ __forceinline__ double dpp_bcast(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)dpp_bcast<BC>((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)dpp_bcast<BC>((int)(uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// 1 / x in fp64: hardware estimate and one Newton step (a few ulps).
__device__ __forceinline__ double rcp_nr(double x) {
  const double r = __builtin_amdgcn_rcp(x);
  return __builtin_fma(r, __builtin_fma(-x, r, 1.0), r);
}

// 1.0 where c holds, else 0.0 (one select: the low word is zero in both).
// fma(x, gate(c), y) is c ? x + y : y for finite x, with x + y rounded once.
__device__ __forceinline__ double gate(bool c) {
  return __hiloint2double(c ? 0x3ff00000 : 0, 0);
}

// lane ^ M through the LDS crossbar, for ints and doubles.
template <int M>
__device__ __forceinline__ int lane_xor_ds_i(int v) {
  return __float_as_int(lane_xor_ds<M>(__int_as_float(v)));
}
template <int M>
__device__ __forceinline__ double lane_xor_ds_d(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)lane_xor_ds_i<M>((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)lane_xor_ds_i<M>((int)(uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive segmented scan over the G lanes of a group in lane order, by DPP
// steps: (f, s) of the lanes up to this one combined as in block_seg_carry.
template <int G>
__device__ __forceinline__ void group_seg_incl(int& f, double& s, int gl) {
  auto step = [&](double sp, int fp) {
    s = __builtin_fma(sp, gate(f == 0), s);  // f ? s : sp + s
    f |= fp;
  };
  auto shr = [&](auto tag) {
    constexpr int N = decltype(tag)::value;
    double sp = dpp_shr<N>(s);
    int fp = dpp_shr<N>(f);
    if (G < 16 && gl < N) {  // two groups share a row
      sp = 0.0;
      fp = 0;
    }
    step(sp, fp);
  };
  shr(std::integral_constant<int, 1>());
  shr(std::integral_constant<int, 2>());
  shr(std::integral_constant<int, 4>());
  if constexpr (G >= 16) shr(std::integral_constant<int, 8>());
  if constexpr (G >= 32) step(dpp_bcast<15>(s), dpp_bcast<15>(f));
  if constexpr (G >= 64) step(dpp_bcast<31>(s), dpp_bcast<31>(f));
}

// Exclusive segmented carry over the G lanes of a group: the combination of
// the aggregates (f, s) of the lanes before this one (REV = false) or after
// it (REV = true; the group's lanes mirrored, scanned, mirrored back).
template <int G, bool REV>
__device__ __forceinline__ double group_seg_carry_dpp(bool f, double s, int gl) {
  int fi = f ? 1 : 0;
  if constexpr (REV) {  // the mirror through the LDS crossbar
    s = lane_xor_ds_d<G - 1>(s);
    fi = lane_xor_ds_i<G - 1>(fi);
  }
  // scan and shift in physical lane order (mirrored order for REV)
  group_seg_incl<G>(fi, s, gl);
  double ex = __shfl_up(s, 1, G);
  if (gl == 0) ex = 0.0;
  if constexpr (REV) ex = lane_xor_ds_d<G - 1>(ex);
  return ex;
}

// Exclusive segmented scan over the G lanes of a group (see block_seg_carry):
// returns the combination of the aggregates (f, s) of the lanes before this
// one (REV = false) or after it (REV = true).
template <int G, bool REV>
__device__ __forceinline__ double group_seg_carry(bool f, double s, int gl) {
  int fi = f ? 1 : 0;
#pragma unroll
  for (int o = 1; o < G; o <<= 1) {
    const double s2 = REV ? __shfl_down(s, o, G) : __shfl_up(s, o, G);
    const int f2 = REV ? __shfl_down(fi, o, G) : __shfl_up(fi, o, G);
    const bool valid = REV ? (gl + o < G) : (gl >= o);
    if (valid) {
      if (!fi) s = s2 + s;
      fi |= f2;
    }
  }
  double ex = REV ? __shfl_down(s, 1, G) : __shfl_up(s, 1, G);
  if (REV ? gl == G - 1 : gl == 0) ex = 0.0;
  return ex;
}

// Exclusive sum over the G lanes of a group: of the lanes before this one
// (REV = false) or after it (REV = true; mirrored, scanned, mirrored back).
// The same additions in the same order as group_seg_carry_dpp without
// segment starts, without its flag bookkeeping.  *total (REV = false): the
// group's sum (the last lane's inclusive value) in every lane.
template <int G, bool REV>
__device__ __forceinline__ double group_excl_sum(double s, int gl, double* total = nullptr) {
  if constexpr (REV) s = lane_xor_ds_d<G - 1>(s);
  auto shr = [&](auto tag) {
    constexpr int N = decltype(tag)::value;
    double sp = dpp_shr<N>(s);
    if (G < 16 && gl < N) sp = 0.0;  // two groups share a row
    s = sp + s;
  };
  shr(std::integral_constant<int, 1>());
  shr(std::integral_constant<int, 2>());
  shr(std::integral_constant<int, 4>());
  if constexpr (G >= 16) shr(std::integral_constant<int, 8>());
  if constexpr (G >= 32) s = dpp_bcast<15>(s) + s;
  if constexpr (G >= 64) s = dpp_bcast<31>(s) + s;
  double ex = __shfl_up(s, 1, G);
  if (gl == 0) ex = 0.0;
  if constexpr (REV) ex = lane_xor_ds_d<G - 1>(ex);
  if constexpr (!REV) {
    if (total != nullptr) *total = __shfl(s, G - 1, G);
  }
  return ex;
}

// Group argmax of (value, key): larger value wins, equal values -> smaller
// key; every lane of the group gets the winner.
template <int G>
__device__ __forceinline__ int group_argmax(double v, int key, double* best_out) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) {
    const double v2 = xshfl(v, o);
    const int k2 = xshfl(key, o);
    if (v2 > v || (v2 == v && k2 < key)) {
      v = v2;
      key = k2;
    }
  }
  *best_out = v;
  return key;
}

// The same where keys increase with the lane: the key of the first lane of
// the group holding the maximum (a max reduction, a ballot, one read).
template <int G>
__device__ __forceinline__ int group_argmax_first(double v, int key, double* best_out) {
  double m = v;
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) m = fmax(m, xshfl(m, o));
  *best_out = m;
  const uint64_t at = (uint64_t)__ballot(v == m);
  if constexpr (G == 64) {
    return __builtin_amdgcn_readlane(key, __builtin_ctzll(at));
  } else {
    const int base = (int)(threadIdx.x & 63u) & ~(G - 1);
    const uint32_t mine = (uint32_t)(at >> base) & (uint32_t)((1ull << G) - 1ull);
    return __shfl(key, base + __builtin_ctz(mine), 64);
  }
}

// The same argmax in two reductions: the group maximum of the value, then
// the smallest key among the lanes holding it.
template <int G>
__device__ __forceinline__ int group_argmax2(double v, int key, double* best_out) {
  double mx = v;
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) mx = fmax(mx, xshfl(mx, o));
  int k = v == mx ? key : 0x7fffffff;
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) k = min(k, xshfl(k, o));
  *best_out = mx;
  return k;
}

// Sorted value at group-uniform position pos.
template <int E, int G>
__device__ __forceinline__ float wave_at(const float (&y)[E], int pos) {
  float v = y[0];
#pragma unroll
  for (int r = 1; r < E; ++r)
    if ((pos % E) == r) v = y[r];
  return __shfl(v, pos / E, G);
}

// NT: nontemporal 128-bit access for whole float4s (streams read or written
// once; ORQ's first read is not one: it reads its bucket again from cache)
// INB: the vector is known to lie inside the gradient (no bounds tests).
template <int VEC, bool NT = false, bool INB = false>
__device__ __forceinline__ void load_vec(const float* __restrict__ a,
                                         int64_t i, int64_t n, float (&x)[VEC]) {
  if constexpr (VEC == 4 && INB) {
    const float4 v = NT ? load4_nt(a + i) : *reinterpret_cast<const float4*>(a + i);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  } else if constexpr (VEC == 4) {
    const float4 v = (NT && i + 4 <= n) ? load4_nt(a + i) : load4(a, i, n);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  } else {
    if (i + VEC <= n) {
      if constexpr (VEC == 2) {
        const float2 v = *reinterpret_cast<const float2*>(a + i);
        x[0] = v.x; x[1] = v.y;
      } else {
        x[0] = a[i];
      }
    } else {
#pragma unroll
      for (int c = 0; c < VEC; ++c) x[c] = (i + c < n) ? a[i + c] : 0.f;
    }
  }
}

template <int VEC, bool NT = false, bool INB = false>
__device__ __forceinline__ void store_vec(float* __restrict__ a, int64_t i,
                                          int64_t n, const float (&x)[VEC]) {
  if constexpr (VEC == 4 && INB) {
    if (NT) store4_nt(a + i, make_float4(x[0], x[1], x[2], x[3]));
    else *reinterpret_cast<float4*>(a + i) = make_float4(x[0], x[1], x[2], x[3]);
  } else if constexpr (VEC == 4) {
    if (NT && i + 4 <= n) store4_nt(a + i, make_float4(x[0], x[1], x[2], x[3]));
    else store4(a, i, n, make_float4(x[0], x[1], x[2], x[3]));
  } else {
    if (i + VEC <= n) {
      if constexpr (VEC == 2) *reinterpret_cast<float2*>(a + i) = make_float2(x[0], x[1]);
      else a[i] = x[0];
    } else {
#pragma unroll
      for (int c = 0; c < VEC; ++c) if (i + c < n) a[i + c] = x[c];
    }
  }
}

// At most 128 VGPRs (4 waves per SIMD): the recursive-bisection variant
// would take 132 and run at 3 (ORQ-9 by bisection on 100M: 2.20 -> 1.94 ms
// at 4 with 16 bytes per lane spilled); the others fit without spilling.
// FULL: every bucket of the launch holds D values (a short last bucket runs
// in a launch of its own), so no value needs a bounds test.  Buckets
// b0 .. nb-1.
template <int SCHEME, int BITS, int D, bool BISECT, bool FULL>
__global__ __launch_bounds__(kGroupThreads, 4)
void k_wave_sort_quant(
    int64_t n, int64_t b0, int64_t nb, const float* __restrict__ g, float* __restrict__ e,
    uint32_t k0, uint32_t k1, uint32_t step, int L, int flags, float clip_sigma,
    uint8_t* __restrict__ codes, float* __restrict__ meta, int64_t code_bytes,
    uint32_t A4, int W, int redo) {
  constexpr int E = WaveCfg<D>::E;
  constexpr int G = WaveCfg<D>::G;
  constexpr int VEC = 4;
  constexpr int NQ = E / VEC;
  const int lane = threadIdx.x % G;  // lane within the bucket's group
  // With one bucket per wave the index is wave-uniform: as a scalar it puts
  // every address in the scalar-base + lane-offset form, so no 64-bit
  // per-lane address has to live (and spill) from the loads to the stores.
  const int64_t bucket = [&] {
    const int64_t bk = b0 + (int64_t)blockIdx.x * (kGroupThreads / G) + threadIdx.x / G;
    if constexpr (G == 64) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bk);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)bk >> 32));
      return (int64_t)(((uint64_t)hi << 32) | lo);
    } else {
      return bk;
    }
  }();
  if (bucket >= nb) return;  // whole groups leave together
  // redo: only the buckets the sort-free BinGrad-b kernel marked with NaN
  // levels (group-uniform)
  if constexpr (SCHEME == BIN_OPT) {
    if (redo && meta[2 * bucket] == meta[2 * bucket]) return;
  }
  const int64_t base = bucket * D;
  const int nj = FULL ? D : (int)((n - base) < D ? (n - base) : D);
  // whole buckets address their values as the base of the wave's first
  // bucket (a scalar: the wave's buckets are consecutive) + a 32-bit offset
  const int64_t wbase = [&] {
    const int64_t wb = (b0 + (int64_t)blockIdx.x * (kGroupThreads / G) +
                        (int64_t)(threadIdx.x / 64) * (64 / G)) * D;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)wb);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)wb >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
  }();
  const float* const gB = g + wbase;
  float* const eB = e == nullptr ? nullptr : e + wbase;
  const uint32_t goff = (uint32_t)(((threadIdx.x & 63) / G) * D);  // group in wave
  auto off = [&](int q) { return goff + (uint32_t)(VEC * (lane + G * q)); };

  // ---- 1. load p = g (+ e), element order --------------------------------
  float p[E];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int64_t i = base + (int64_t)VEC * (lane + G * q);
    float x[VEC];
    if constexpr (FULL) load_vec<VEC, SCHEME == BIN_OPT, true>(gB, off(q), n, x);
    else load_vec<VEC, SCHEME == BIN_OPT, false>(g, i, n, x);
    if (e != nullptr) {
      float r[VEC];
      if constexpr (FULL) load_vec<VEC, SCHEME == BIN_OPT, true>(eB, off(q), n, r);
      else load_vec<VEC, SCHEME == BIN_OPT, false>(e, i, n, r);
#pragma unroll
      for (int c = 0; c < VEC; ++c) x[c] = x[c] + r[c];
    }
#pragma unroll
    for (int c = 0; c < VEC; ++c) p[VEC * q + c] = x[c];
  }
  auto epos = [&](int m) { return VEC * (lane + G * (m / VEC)) + (m % VEC); };

  // ---- 2. clip (ORQ) -----------------------------------------------------
  const bool clip = (flags & GQ_FLAG_CLIP) != 0;
  float C = __builtin_inff();
  if (SCHEME == ORQ && clip) {
    Sum2 sq{0.0, 0.0};
#pragma unroll
    for (int m = 0; m < E; ++m)
      if (epos(m) < nj) two_sum_add(sq, (double)p[m] * (double)p[m]);
    sq = group_sum2<G>(sq);
    const double sigma = sqrt((sq.s + sq.c) / (double)nj);
    C = (float)((double)clip_sigma * sigma);
  }
  // (C = +inf without clipping: the median of x, -C, C is then x)
  auto clipped = [&](float x) {
    if constexpr (SCHEME == ORQ) return __builtin_amdgcn_fmed3f(x, -C, C);
    else return x;
  };

  // ---- 3. sort in registers (canonical +0, +inf padding) -----------------
  float y[E];
#pragma unroll
  for (int m = 0; m < E; ++m) {
    // x + 0 is x, except -0 + 0 = +0 (denormals are kept)
    y[m] = epos(m) < nj ? clipped(p[m]) + 0.f : __builtin_inff();
  }
  flip_bitonic<E, D>(y, nullptr, lane);

  const int r0 = lane * E;
  float y_next_run = __shfl_down(y[0], 1, G);
  if (lane == G - 1) y_next_run = __builtin_inff();

  float lvl_a = 0.f, lvl_b = 0.f, thr = 0.f;
  bool no_split = false;
  // ORQ: each group's levels, ascending, +inf past the current count
  __shared__ float lvt[kGroupThreads / G][16];

  if constexpr (SCHEME == BIN_OPT) {
    // ---- 4a. best split -------------------------------------------------
    // (from the first value: 0 + y would cost an add; y is never -0)
    double tot = r0 < nj ? (double)y[0] : 0.0;
#pragma unroll
    for (int m = 1; m < E; ++m)
      if (r0 + m < nj) tot = tot + (double)y[m];
    // the sum of the lanes before this one (P's start), the bucket sum S and
    // what follows this lane's values, S - (pre + tot) (Q's start: its
    // rounding differs from a suffix sum's by a few ulps of S, which moves F
    // by far less than the tie tolerance)
    double Sg;
    const double pre = group_excl_sum<G, false>(tot, lane, &Sg);
    const double suf = Sg - (pre + tot);
    // F(k) = P^2/k + Q^2/(n-k) at every split between distinct values.  With
    // mu = S/n and the centred sum C = P - k mu, F(k) = S^2/n + n D(k),
    // D(k) = C^2 / (k (n-k)), so F and D peak at the same splits.  D is
    // screened in fp32 (C from fp64 running sums, scaled by a power of two
    // so |C| <= 2d: relative error < 1e-6, below 1e-5 of the maximum), then
    // F is evaluated in fp64 only at splits whose D is within 1e-5 of the
    // screen's maximum, with P and Q = S - P summed from the lane's carries
    // in the order of the values.  The screen keeps the maximum and every
    // near tie; the fp64 values take refined reciprocals (a few ulps):
    // splits closer than that are ties, where either is correct.
    const float amax = fmaxf(fabsf(wave_at<E, G>(y, 0)), fabsf(wave_at<E, G>(y, nj - 1)));
    int ex = 0;
    frexpf(amax, &ex);
    const double sc = ldexp(1.0, -ex);
    const double mu = Sg / (double)nj;
    // (branch-free: every slot evaluated, -1 selected where no split lies;
    // k (n - k) = k0 n0 + m (n0 - k0 - m) from the lane's first split k0,
    // n0 = n - k0, exact in fp32 for n <= 4096)
    float Fa[E];
    float fmax32 = -1.f;
    {
      float kf0 = (float)(r0 + 1), nkf0 = (float)(nj - r0 - 1);
      // (opaque: otherwise folded back into conversions per slot)
      asm volatile("" : "+v"(kf0), "+v"(nkf0));
      const float kkA = kf0 * nkf0, kkB = nkf0 - kf0;
      double Cs = pre - (double)r0 * mu;
#pragma unroll
      for (int m = 0; m < E; ++m) {
        if (r0 + m < nj) Cs = Cs + ((double)y[m] - mu);
        const float yk = (m + 1 < E) ? y[m + 1] : y_next_run;
        const float c32 = (float)(Cs * sc);
        const float kk = m == 0 ? kkA : __builtin_fmaf((float)m, kkB - (float)m, kkA);
        const float f = c32 * c32 * __builtin_amdgcn_rcpf(kk);
        Fa[m] = (r0 + m + 1 < nj && y[m] < yk) ? f : -1.f;
        fmax32 = fmaxf(fmax32, Fa[m]);
      }
    }
    // (as integers: the order of the bit patterns of floats >= 0, and -1
    // below them all)
    fmax32 = __int_as_float(group_reduce<G>(__float_as_int(fmax32),
                                            [](int a, int b) { return a > b ? a : b; }));
    const float screen = fmax32 * (1.0f - 1e-5f);
    double best = -1.0;
    int bestk = 0x7fffffff;
    double bestP = 0.0;  // the sum below this lane's best split
    // Four or more groups in a wave meet their candidates in different
    // slots; where no lane holds two, each lane sums for its own slot in one
    // pass (the other values add 0.0, which leaves the sums as they are).
    bool done = false;
    if constexpr (G <= 16) {
      int nc = 0, mc = 0;
#pragma unroll
      for (int m = 0; m < E; ++m) {
        const bool c = Fa[m] >= screen;
        nc += c ? 1 : 0;
        mc = c ? m : mc;
      }
      if (__ballot(nc > 1) == 0ull) {
        done = true;
        if (nc == 1) {
          double P = pre, Q = suf;
#pragma unroll
          for (int i = 0; i < E; ++i) {
            float v = y[i];
            asm volatile("" : "+v"(v));
            P = P + (i <= mc ? (double)v : 0.0);  // (slot mc has a split: i < nj)
          }
#pragma unroll
          for (int i = E - 1; i >= 0; --i) {
            float v = y[i];
            asm volatile("" : "+v"(v));
            Q = Q + (i > mc && r0 + i < nj ? (double)v : 0.0);
          }
          const int k = r0 + mc + 1;
          best = P * P * rcp_nr((double)k) + Q * Q * rcp_nr((double)(nj - k));
          bestk = k;
          bestP = P;
        }
      }
    }
#pragma unroll
    for (int m = 0; m < E; ++m) {
      if (!done && Fa[m] >= screen) {  // (screen > -1: no slot without a split)
        // (the values reread as opaque floats: no fp64 copies kept live)
        double P = pre, Q = suf;
#pragma unroll
        for (int i = 0; i < E; ++i) {
          float v = y[i];
          asm volatile("" : "+v"(v));
          if (i <= m && r0 + i < nj) P = P + (double)v;
        }
#pragma unroll
        for (int i = E - 1; i > m; --i) {
          float v = y[i];
          asm volatile("" : "+v"(v));
          if (r0 + i < nj) Q = Q + (double)v;
        }
        const int k = r0 + m + 1;
        const double F = P * P * rcp_nr((double)k) + Q * Q * rcp_nr((double)(nj - k));
        if (F > best) {
          best = F;
          bestk = k;
          bestP = P;
        }
      }
    }
    // the largest F, then the smallest split (lanes hold increasing splits);
    // where no group has candidates in more than one lane (the usual case)
    // the candidate lane's own best
    double bestF;
    int kstar;
    {
      const uint64_t cl = (uint64_t)__ballot(best >= 0.0);
      const int gbase = (int)(threadIdx.x & 63u) & ~(G - 1);
      const uint64_t mine = G == 64 ? cl : (cl >> gbase) & ((1ull << (G & 63)) - 1ull);
      if (__ballot((mine & (mine - 1ull)) != 0ull) == 0ull) {
        const int src = gbase + (mine ? __builtin_ctzll(mine) : 0);
        kstar = __shfl(bestk, src, 64);
        bestF = mine ? __shfl(best, src, 64) : -1.0;
      } else {
        kstar = group_argmax_first<G>(best, bestk, &bestF);
      }
    }
    if (bestF < 0.0) {
      no_split = true;
      thr = wave_at<E, G>(y, 0);
      lvl_a = lvl_b = thr;
    } else {
      thr = wave_at<E, G>(y, kstar);
      // the cluster sums: the prefix sum at the split (from the lane that
      // holds its last lower value) and the rest of the bucket sum; where a
      // sum is small against the bucket's magnitude (cancellation) both are
      // recomputed with compensated sums
      const double Ps = __shfl(bestP, (kstar - 1) / E, G);
      const double Stot = Sg;
      const double tiny = 0x1p-20 * (double)amax * (double)nj;
      double slo = Ps, shi = Stot - Ps;
      if (fabs(slo) < tiny || fabs(shi) < tiny) {
        Sum2 lo{0.0, 0.0}, hi{0.0, 0.0};
#pragma unroll
        for (int m = 0; m < E; ++m) {
          const int pos = r0 + m;
          if (pos < kstar) two_sum_add(lo, (double)y[m]);
          else if (pos < nj) two_sum_add(hi, (double)y[m]);
        }
        lo = group_sum2<G>(lo);
        hi = group_sum2<G>(hi);
        slo = lo.s + lo.c;
        shi = hi.s + hi.c;
      }
      lvl_a = (float)(slo / (double)kstar);
      lvl_b = (float)(shi / (double)(nj - kstar));
    }
    if (lane == 0) {
      meta[2 * bucket + 0] = lvl_a;
      meta[2 * bucket + 1] = lvl_b;
    }
  } else {
    // ---- 4b. ORQ greedy levels --------------------------------------------
    // The levels live in the group's LDS row T, ascending, +inf past the
    // current count.  Each sorted value keeps its segment's end points
    // (a, b) (a = the last level <= y; the top segment, y >= max, has
    // a = b = max) and, for the bisection, the segment's index; inserting c
    // into (a0, b0) splits it into (a0, c), (c, b0).  One level per step
    // (greedy), or with GQ_FLAG_BISECT one per segment per round (recursive
    // bisection).
    float* T = lvt[threadIdx.x / G];
    const float ymin = wave_at<E, G>(y, 0), ymax = wave_at<E, G>(y, nj - 1);
    const bool flat = !(ymin < ymax);
    for (int j = lane; j < 16; j += G)
      T[j] = flat ? (j < L ? ymin : __builtin_inff())
                  : (j == 0 ? ymin : (j == 1 ? ymax : __builtin_inff()));
    int cnt = flat ? L : 2;
    // the +inf padding past the bucket's end becomes ymax here: it then sits
    // in the top segment with y - a = b - y = 0 and is never a candidate
#pragma unroll
    for (int m = 0; m < E; ++m) y[m] = r0 + m < nj ? y[m] : ymax;
    int seg[BISECT ? E : 1];
    float a_of[E], b_of[E];
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const bool top = y[m] >= ymax;
      if constexpr (BISECT) seg[m] = top ? 1 : 0;
      a_of[m] = top ? ymax : ymin;
      b_of[m] = ymax;
    }
    // a segment identifier: its index, or the bits of its lower end (the
    // levels are distinct values)
    auto sid = [&](int m) {
      if constexpr (BISECT) return seg[m];
      else return __float_as_int(a_of[m]);
    };
    while (cnt < L) {
      int seg_prev = __shfl_up(sid(E - 1), 1, G);
      const bool first_lane = lane == 0;
      int seg_next = __shfl_down(sid(0), 1, G);
      const bool last_lane = lane == G - 1 || r0 + E >= nj;
      // (b - y) once per step, (y - a) at each use; both exact in fp64
      double dB[E];
#pragma unroll
      for (int m = 0; m < E; ++m) dB[m] = (double)b_of[m] - (double)y[m];
      auto va = [&](int m) { return (double)y[m] - (double)a_of[m]; };
      auto vb = [&](int m) { return dB[m]; };
      auto head = [&](int m) {
        return m == 0 ? (first_lane || seg_prev != sid(0)) : sid(m) != sid(m - 1);
      };
      auto tail = [&](int m) {
        return m == E - 1 ? (last_lane || seg_next != sid(E - 1)) : sid(m) != sid(m + 1);
      };
      // restart ? v : s + v; the greedy kernel takes it as one fma with a
      // 1.0/0.0 factor (one select instead of two), the bisection kernel
      // (more live state) as selects, which need no register pair for the
      // factor
      auto acc = [](double s, bool restart, double v) {
        if constexpr (BISECT) return restart ? v : s + v;
        else return __builtin_fma(s, gate(!restart), v);
      };
      // this lane's partial sums (branch-free), then the group's carries
      int fa = 0, fb = 0;
      // (from 0, the first value's sum is the value itself)
      double sa = va(0), sb = vb(E - 1);
      fa = head(0) ? 1 : 0;
      fb = tail(E - 1) ? 1 : 0;
#pragma unroll
      for (int m = 1; m < E; ++m) {
        const bool h = head(m);
        sa = acc(sa, h, va(m));
        fa |= h ? 1 : 0;
      }
#pragma unroll
      for (int m = E - 2; m >= 0; --m) {
        const bool t = tail(m);
        sb = acc(sb, t, vb(m));
        fb |= t ? 1 : 0;
      }
      const double ca = group_seg_carry_dpp<G, false>(fa != 0, sa, lane);
      const double cb = group_seg_carry_dpp<G, true>(fb != 0, sb, lane);
      double best = -1.0;
      int bestk = 0x7fffffff;
      // Gs[m]: first the sum of (b - y) over the values after m in m's
      // segment, then m's gain G (-1 for a value that is no candidate)
      double Gs[E];
      {
        double run = cb;  // >= 0
#pragma unroll
        for (int m = E - 1; m >= 0; --m) {
          const bool t = tail(m);
          if constexpr (BISECT) {
            Gs[m] = t ? 0.0 : run;
            run = acc(run, t, vb(m));
          } else {  // one factor for both
            const double k = gate(!t);
            Gs[m] = run * k;
            run = __builtin_fma(run, k, vb(m));
          }
        }
        double A = ca;
#pragma unroll
        for (int m = 0; m < E; ++m) {
          const double v = va(m);
          A = acc(A, head(m), v);
          const int pos = r0 + m;
          const float yv = y[m];
          const float ynext = (m + 1 < E) ? y[m + 1] : y_next_run;
          // strictly inside a segment other than the top one (a value of
          // the top segment equals its lower end, ymax), the last of a run
          // of equal values
          const bool cand = pos < nj && yv > a_of[m] && (pos + 1 >= nj || ynext != yv);
          // (b - c) A + (c - a) B, with b - c and c - a exact in fp64
          if constexpr (BISECT) {
            const double Gv = cand ? vb(m) * A + v * Gs[m] : -1.0;
            const bool better = Gv > best;
            best = better ? Gv : best;
            bestk = better ? pos : bestk;
            Gs[m] = Gv;
          } else {
            const double Gv = vb(m) * A + v * Gs[m];
            const bool better = cand && Gv > best;
            best = better ? Gv : best;
            bestk = better ? pos : bestk;
          }
        }
      }
      // insert c after every level below it (levels stay ascending; c lies
      // strictly inside a segment, so no level equals it) and update the
      // segment state of every value
      auto insert_level = [&](float c) {
        const int ins = lds_rank16(T, c);
        constexpr int NJ = (16 + G - 1) / G;
        float old[NJ];
#pragma unroll
        for (int t = 0; t < NJ; ++t) {
          const int j = lane + G * t;
          old[t] = (j >= 1 && j < 16) ? T[j - 1] : 0.f;
        }
#pragma unroll
        for (int t = 0; t < NJ; ++t) {
          const int j = lane + G * t;
          if (j < 16 && j >= ins && j <= cnt) T[j] = j == ins ? c : old[t];
        }
#pragma unroll
        for (int m = 0; m < E; ++m) {
          const bool split = a_of[m] < c && c < b_of[m];
          const bool up = y[m] >= c;
          a_of[m] = (split && up) ? c : a_of[m];
          b_of[m] = (split && !up) ? c : b_of[m];
          if constexpr (BISECT) seg[m] += up ? 1 : 0;
        }
        ++cnt;
      };
      auto fill_with_max = [&]() {
        // fewer distinct values than levels: repeat the maximum
        for (int j = lane; j < 16; j += G)
          if (j >= cnt && j < L) T[j] = ymax;
        cnt = L;
      };
      if constexpr (!BISECT) {
        double bestG;
        const int kstar = group_argmax_first<G>(best, bestk, &bestG);
        if (bestG < 0.0) fill_with_max();
        else insert_level(wave_at<E, G>(y, kstar));
      } else {
        // Recursive bisection: the best value of every segment, segment j
        // kept by lane j mod G in slot j / G; then the round's candidates
        // are inserted, all of them or (when they would pass L levels) the
        // largest gains first, equal gains by position.
        constexpr int NSL = (15 + G - 1) / G;
        double sg[NSL];
        int sk[NSL];
#pragma unroll
        for (int t = 0; t < NSL; ++t) {
          sg[t] = -1.0;
          sk[t] = 0x7fffffff;
        }
        const int nseg = cnt - 1;
        for (int j = 0; j < nseg; ++j) {
          double bj = -1.0;
          int kj = 0x7fffffff;
#pragma unroll
          for (int m = 0; m < E; ++m)
            if (seg[m] == j && Gs[m] > bj) {
              bj = Gs[m];
              kj = r0 + m;
            }
          double bg;
          const int kg = group_argmax<G>(bj, kj, &bg);
#pragma unroll
          for (int t = 0; t < NSL; ++t)
            if (j == lane + G * t && bg >= 0.0) {
              sg[t] = bg;
              sk[t] = kg;
            }
        }
        int have = 0;
#pragma unroll
        for (int t = 0; t < NSL; ++t) have += sg[t] >= 0.0 ? 1 : 0;
        have = group_sum_i<G>(have);
        if (have == 0) {
          fill_with_max();
        } else {
          const int take = have < L - cnt ? have : L - cnt;
          for (int t2 = 0; t2 < take; ++t2) {
            double lb = -1.0;
            int lk = 0x7fffffff;
#pragma unroll
            for (int t = 0; t < NSL; ++t)
              if (sg[t] > lb || (sg[t] == lb && sk[t] < lk)) {
                lb = sg[t];
                lk = sk[t];
              }
            double gb;
            const int kb = group_argmax<G>(lb, lk, &gb);
#pragma unroll
            for (int t = 0; t < NSL; ++t)
              if (sk[t] == kb) {
                sg[t] = -1.0;
                sk[t] = 0x7fffffff;
              }
            insert_level(wave_at<E, G>(y, kb));
          }
        }
      }
    }
    for (int j = lane; j < L; j += G) meta[bucket * L + j] = T[j];
  }

  if (codes == nullptr) return;  // levels only

  // ---- 5. codes, packing, residual (element order) ----------------------
  // ORQ reads its bucket again here (from cache in practice) rather than
  // holding p through the level search: fewer live registers, more waves.
  if constexpr (SCHEME == ORQ) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int64_t i = base + (int64_t)VEC * (lane + G * q);
      float x[VEC];
      if constexpr (FULL) load_vec<VEC, false, true>(gB, off(q), n, x);
      else load_vec<VEC, false, false>(g, i, n, x);
      if (e != nullptr) {
        float r[VEC];
        if constexpr (FULL) load_vec<VEC, false, true>(eB, off(q), n, r);
        else load_vec<VEC, false, false>(e, i, n, r);
#pragma unroll
        for (int c = 0; c < VEC; ++c) x[c] = x[c] + r[c];
      }
#pragma unroll
      for (int c = 0; c < VEC; ++c) p[VEC * q + c] = x[c];
    }
  }
  uint32_t dfield[BITS == 0 ? NQ : 1];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int64_t i0 = base + (int64_t)VEC * (lane + G * q);
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (SCHEME == ORQ) {
      // random words, or (nearest) words whose u is exactly 1/2: the value
      // then rounds up iff q > 1/2
      w = make_uint4(kHalfWord, kHalfWord, kHalfWord, kHalfWord);
      if (!(flags & GQ_FLAG_NEAREST)) {
        const uint64_t ctr = (uint64_t)i0 >> 2;
        w = philox4x32_10(k0, k1, (uint32_t)ctr, (uint32_t)(ctr >> 32), step, 0u);
      }
    }
    // BITS-bit codes, or (dense) 4-bit digits turned into one base-L
    // number at the store
    uint32_t field = 0u;
    float r[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      const int m = VEC * q + c;
      const int64_t i = i0 + c;
      const bool real = FULL || i < n;
      uint32_t code = 0u;
      float xh = 0.f;
      if constexpr (SCHEME == BIN_OPT) {
        code = (!no_split && p[m] >= thr) ? 1u : 0u;
        xh = code ? lvl_b : lvl_a;
      } else {
        // the levels around x by binary search in the group's LDS row: a
        // value on a level takes it (the first equal one); otherwise it
        // rounds between the levels below and above
        const float* T = lvt[threadIdx.x / G];
        const float x = clipped(p[m]);
        const int above = lds_rank16(T, x);  // levels below x
        const float hi = T[above];
        const float lo = T[above > 0 ? above - 1 : 0];
        const int sub = (int)(i & 3);
        const uint32_t word = sub == 0 ? w.x : sub == 1 ? w.y : sub == 2 ? w.z : w.w;
        const float qf = (x - lo) / (hi - lo);
        const bool up = u24(word) < qf;
        const bool on = hi == x;
        code = (uint32_t)(on ? above : above - 1 + (up ? 1 : 0));
        xh = on ? x : (up ? hi : lo);
      }
      if (!real) code = 0u;
      field |= code << ((BITS == 0 ? 4 : BITS) * c);
      r[c] = p[m] - xh;
    }
    if constexpr (BITS == 0) dfield[q] = field;
    else store_chunk<BITS, VEC>(codes, i0, lane, field, code_bytes);
    if constexpr (FULL) {
      if (e != nullptr) store_vec<VEC, true, true>(eB, off(q), n, r);
    } else {
      if (e != nullptr && i0 < n) store_vec<VEC, true, false>(e, i0, n, r);
    }
  }
  // Dense fields are stored once the values and levels are dead.  Dense ORQ
  // runs with d >= 512 only, so here a bucket is one wave.
  if constexpr (BITS == 0 && G == 64) {
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      store_dense_chunk(codes, base + (int64_t)VEC * G * q,
                        nibbles_to_base(dfield[q], L), A4, W, code_bytes);
  }
}

template <int SCHEME, int BITS, int D>
int launch_sort_one(int64_t n, const float* g, float* e, uint64_t seed,
                    uint32_t step, int L, int flags, float clip_sigma,
                    uint8_t* codes, float* meta, int64_t code_bytes,
                    uint32_t A4, int W, int redo, hipStream_t st) {
  const int64_t nb = (n + D - 1) / D;
  if (BITS == 0 && D < 512) return (int)hipErrorInvalidValue;  // dense: d >= 512
  if constexpr (D <= 512) {
    constexpr int per_block = kGroupThreads / WaveCfg<D>::G;
    // the whole buckets, then (one block) the short last one
    const int64_t nfull = n / D;
    auto go = [&](auto kern, int64_t first, int64_t end) {
      const int64_t blocks = (end - first + per_block - 1) / per_block;
      if (blocks > 0)
        hipLaunchKernelGGL(kern, dim3((uint32_t)blocks), dim3(kGroupThreads), 0, st,
                           n, first, end, g, e, (uint32_t)seed, (uint32_t)(seed >> 32),
                           step, L, flags, clip_sigma, codes, meta, code_bytes,
                           A4, W, redo);
    };
    const bool bisect = SCHEME == ORQ && (flags & GQ_FLAG_BISECT) != 0;
    if (bisect) {
      if constexpr (SCHEME == ORQ) {
        go(k_wave_sort_quant<SCHEME, BITS, D, true, true>, 0, nfull);
        go(k_wave_sort_quant<SCHEME, BITS, D, true, false>, nfull, nb);
      }
    } else {
      go(k_wave_sort_quant<SCHEME, BITS, D, false, true>, 0, nfull);
      go(k_wave_sort_quant<SCHEME, BITS, D, false, false>, nfull, nb);
    }
  } else {
    // the redo pass: one workgroup per 64 buckets (see k_sort_quant)
    const int64_t grid = redo ? (nb + 63) / 64 : nb;
    hipLaunchKernelGGL((k_sort_quant<SCHEME, BITS, D>), dim3((uint32_t)grid),
                       dim3(SortCfg<D>::T), 0, st, n, g, e, (uint32_t)seed,
                       (uint32_t)(seed >> 32), step, L, flags, clip_sigma, codes,
                       meta, code_bytes, A4, W, redo);
  }
  return (int)hipGetLastError();
}

template <int SCHEME, int BITS>
int sort_dispatch_d(int d, int64_t n, const float* g, float* e, uint64_t seed,
                    uint32_t step, int L, int flags, float clip_sigma,
                    uint8_t* codes, float* meta, int64_t code_bytes,
                    uint32_t A4, int W, hipStream_t st, int redo = 0) {
#define GQ_SCASE(D_)                                                        \
  case D_:                                                                  \
    return launch_sort_one<SCHEME, BITS, D_>(n, g, e, seed, step, L, flags, \
                                             clip_sigma, codes, meta,       \
                                             code_bytes, A4, W, redo, st);
  switch (d) {
    GQ_SCASE(64)
    GQ_SCASE(128)
    GQ_SCASE(256)
    GQ_SCASE(512)
    GQ_SCASE(1024)
    GQ_SCASE(2048)
    GQ_SCASE(4096)
    GQ_SCASE(8192)
    GQ_SCASE(16384)
    GQ_SCASE(32768)
    default:
      return (int)hipErrorInvalidValue;
  }
#undef GQ_SCASE
}

}  // namespace

int launch_sort_quant(const LaunchDesc& L, int64_t n, const float* g, float* e,
                      uint64_t seed, uint32_t step, uint8_t* codes, float* meta,
                      int64_t code_bytes, hipStream_t st) {
  const int flags = L.flags & (GQ_FLAG_CLIP | GQ_FLAG_NEAREST | GQ_FLAG_BISECT);
  if (L.scheme == BIN_OPT) {
    // sort-free split search where it is built, then the sort-based kernel
    // over the buckets it leaves unresolved (marked by NaN levels)
    if (binopt_prune_supported(L.d)) {
      const int rc = launch_binopt_prune(L.d, n, g, e, codes, meta, code_bytes, st);
      if (rc != 0) return rc;
      return sort_dispatch_d<BIN_OPT, 1>(L.d, n, g, e, seed, step, 2, 0, 0.f,
                                         codes, meta, code_bytes, 0u, 0, st, 1);
    }
    return sort_dispatch_d<BIN_OPT, 1>(L.d, n, g, e, seed, step, 2, 0, 0.f,
                                       codes, meta, code_bytes, 0u, 0, st);
  }
#define GQ_ORQ(BITS)                                                          \
  sort_dispatch_d<ORQ, BITS>(L.d, n, g, e, seed, step, L.L, flags,            \
                             L.clip_sigma, codes, meta, code_bytes, L.A4, L.W, \
                             st)
  if (L.dense) return GQ_ORQ(0);
  switch (L.bits) {
    case 1:
      return GQ_ORQ(1);
    case 2:
      return GQ_ORQ(2);
    case 3:
      return GQ_ORQ(3);
    case 4:
      return GQ_ORQ(4);
    default:
      return (int)hipErrorInvalidValue;
  }
#undef GQ_ORQ
}

}  // namespace gq
