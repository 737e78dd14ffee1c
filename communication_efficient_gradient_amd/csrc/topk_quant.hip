// topk_quant.hip — Top-K sparsification combined with quantization ("gradient
// quantization for communication" glossary, §Quantization Schemes: send only
// the largest gradients, combined with quantization; error feedback keeps
// what was not sent).
//
// One wave per bucket of d <= 512 elements; lane l holds the float4 groups
// l + 64 v (v < V = ceil(d / 256)), so the wave reads the bucket with 128-bit
// loads.  Per bucket:
//   1. p = g (+ e); key = the bits of |p| (monotone in |p| for finite values)
//      for real elements, -1 for absent ones; M = max |p|.
//   2. The k = min(K, n_j)-th largest key T, bit by bit from the top: a bit
//      stays set when at least k keys reach the candidate (counts by ballot);
//      the search stops once a single key is left between the bounds.
//   3. Kept: key > T, and the first k - #(key > T) elements with key == T in
//      index order.  Ranks in index order come from per-element ballots
//      (elements before (v, lane, c) are those of earlier v, of lower lanes at
//      the same v, and earlier c in the same group).
//   4. A kept element's slot is its rank among the kept; its index and value
//      go to LDS by slot, lane t codes slot t (the uniform code of
//      gq_quantize with the same Philox word, drawn for kept elements
//      only), and lane w then assembles record word w from the slots that
//      meet it (records are word-aligned).
//   5. Residual e = p - xhat (0 for elements not sent).
// The decoder gives every bucket an LDS row of d floats, adds each payload's
// slots in payload order, and writes the row as alpha * row (+ beta * out).
#include "common.hpp"

namespace gq {
namespace {

constexpr int kWavesPerBlock = 4;

template <int V>
__device__ __forceinline__ int count_ge(const int (&key)[V][4], int t) {
  int c = 0;
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int k = 0; k < 4; ++k) c += __popcll(__ballot(key[v][k] >= t));
  return c;
}

// For a predicate held per element, the number of elements with it set that
// come before each element in index order (index = 4 (lane + 64 v) + c).
template <int V>
__device__ __forceinline__ void rank_before(const bool (&f)[V][4], int (&r)[V][4]) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int prior = 0;  // elements of earlier v
#pragma unroll
  for (int v = 0; v < V; ++v) {
    uint64_t m[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) m[k] = __ballot(f[v][k]);
    int lower = 0;  // same v, lower lanes
#pragma unroll
    for (int k = 0; k < 4; ++k) lower += __popcll(m[k] & lt);
    int own = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      r[v][k] = prior + lower + own;
      own += f[v][k] ? 1 : 0;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) prior += __popcll(m[k]);
  }
}

template <int BITS, int V>
__global__ __launch_bounds__(64 * kWavesPerBlock) void k_topk_quant(
    int64_t n, int64_t nb, int d, int ib, int K, int R,
    const float* __restrict__ g, float* __restrict__ e, uint32_t k0,
    uint32_t k1, uint32_t step, int s, int nearest,
    uint8_t* __restrict__ codes, float* __restrict__ meta) {
  // per slot (kept element, in index order) of the wave's bucket: first its
  // index within the bucket, then its record field; and its value p, then
  // its dequantized value
  __shared__ uint32_t slots_all[kWavesPerBlock][512];
  __shared__ float vals_all[kWavesPerBlock][512];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t bucket = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  const bool live = bucket < nb;  // waves past the end still reach the barrier
  const int64_t base = bucket * d;
  const int nj = live ? (int)((n - base) < d ? (n - base) : d) : 0;
  uint32_t* slot_field = slots_all[wave];
  float* slot_val = vals_all[wave];

  // ---- 1. load, keys, scale -------------------------------------------------
  float4 p[V];
  int key[V][4];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int i = 4 * (lane + 64 * v);  // index within the bucket
    p[v] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < nj) {
      const bool full = i + 4 <= nj;  // nontemporal 128-bit streams
      p[v] = full ? load4_nt(g + base + i) : load4(g, base + i, base + nj);
      if (e != nullptr) {
        const float4 r = full ? load4_nt(e + base + i) : load4(e, base + i, base + nj);
        p[v].x = p[v].x + r.x;
        p[v].y = p[v].y + r.y;
        p[v].z = p[v].z + r.z;
        p[v].w = p[v].w + r.w;
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      key[v][c] = i + c < nj ? (int)__float_as_uint(fabsf(comp(p[v], c))) : -1;
  }
  // absent elements were loaded as 0 and never raise the maximum
  float mloc = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v)
    mloc = fmaxf(mloc, fmaxf(fmaxf(fabsf(p[v].x), fabsf(p[v].y)),
                             fmaxf(fabsf(p[v].z), fabsf(p[v].w))));
  const float M = group_max<64>(mloc);

  // ---- 2. threshold: the k-th largest key -----------------------------------
  // After the round for bit b the k-th largest key lies in [T, T + 2^b), with
  // c_lo keys >= T (c_lo >= kk) and c_hi keys >= T + 2^b (c_hi < kk).  Once
  // that interval holds a single key (c_lo - c_hi = 1) it is the k-th
  // largest: the smallest key >= T.
  const int kk = nj < K ? nj : K;
  int T = 0;
  if (kk > 0) {
    int c_lo = nj, c_hi = 0;
    for (int bit = 30; bit >= 0 && c_lo - c_hi > 1; --bit) {
      const int cand = T | (1 << bit);
      const int c = count_ge<V>(key, cand);
      if (c >= kk) {
        T = cand;
        c_lo = c;
      } else {
        c_hi = c;
      }
    }
    if (c_lo - c_hi == 1) {
      int m = 0x7fffffff;
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (key[v][c] >= T) m = min(m, key[v][c]);
      T = group_reduce<64>(m, [](int a, int b) { return min(a, b); });
    }
  }
  const int above = count_ge<V>(key, T + 1);

  // ---- 3. kept set, 4. slots ------------------------------------------------
  bool tie[V][4], kept[V][4];
  int r[V][4];
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int c = 0; c < 4; ++c) tie[v][c] = kk > 0 && key[v][c] == T;
  rank_before<V>(tie, r);
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      kept[v][c] = kk > 0 && (key[v][c] > T || (tie[v][c] && r[v][c] < kk - above));
  rank_before<V>(kept, r);

  // ---- 5. codes, by slot: lane t codes the kept elements of slots t, t + 64,
  // ... with the Philox word of its element (one draw per kept element)
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (kept[v][c]) {
        slot_field[r[v][c]] = (uint32_t)(4 * (lane + 64 * v) + c);
        slot_val[r[v][c]] = comp(p[v], c);
      }
  __syncthreads();
  const float sf = (float)s;
  const float up = M < 0x1p-96f ? 0x1p96f : 1.0f;
  const float inv = M > 0.f ? sf / (M * up) : 0.f;
  const float delta = M / sf;
  const int fw = ib + BITS;  // slot width
  for (int t = lane; t < kk; t += 64) {
    const uint32_t idx = slot_field[t];
    const uint64_t ctr = (uint64_t)(base + idx) >> 2;
    uint32_t w = kHalfWord;
    if (!nearest) {
      const uint4 r4 = philox4x32_10(k0, k1, (uint32_t)ctr, (uint32_t)(ctr >> 32), step, 0u);
      const uint32_t sub = idx & 3u;
      w = sub == 0 ? r4.x : (sub == 1 ? r4.y : (sub == 2 ? r4.z : r4.w));
    }
    const int ci = up == 1.0f ? uniform_code<false>(slot_val[t], up, inv, sf, w)
                              : uniform_code<true>(slot_val[t], up, inv, sf, w);
    slot_field[t] = idx | (((uint32_t)ci & ((1u << BITS) - 1u)) << ib);
    slot_val[t] = (float)ci * delta;
  }
  __syncthreads();
  float4 xh[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float x[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c] = kept[v][c] ? slot_val[r[v][c]] : 0.f;
    xh[v] = make_float4(x[0], x[1], x[2], x[3]);
  }

  // ---- store: record words, scale, residual ---------------------------------
  if (live) {
    // word w of the record holds bits [32 w, 32 w + 32): the slots that meet
    // it are floor(32 w / fw) .. floor((32 w + 31) / fw), slots >= kk are 0
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes) + bucket * (int64_t)R;
    for (int w = lane; w < R; w += 64) {
      uint32_t word = 0u;
      const int t0 = (32 * w) / fw, t1 = (32 * w + 31) / fw;
      for (int t = t0; t <= t1 && t < kk; ++t) {
        const int off = t * fw - 32 * w;  // bit of slot t inside word w
        const uint32_t f = slot_field[t];
        word |= off >= 0 ? (f << off) : (f >> (-off));
      }
      dst[w] = word;
    }
    if (lane == 0) meta[bucket] = M;
    if (e != nullptr) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int i = 4 * (lane + 64 * v);
        if (i < nj) {
          float4 rr;
          rr.x = p[v].x - xh[v].x;
          rr.y = p[v].y - xh[v].y;
          rr.z = p[v].z - xh[v].z;
          rr.w = p[v].w - xh[v].w;
          if (i + 4 <= nj) store4_nt(e + base + i, rr);
          else store4(e, base + i, base + nj, rr);
        }
      }
    }
  }
}

template <int BITS>
__global__ __launch_bounds__(64 * kWavesPerBlock) void k_topk_deq(
    int64_t n, int64_t nb, int d, int ib, int K, int R, int s, int W,
    PayloadPtrs pp, float alpha, float beta, float* __restrict__ out) {
  __shared__ __align__(16) float row_all[kWavesPerBlock][512];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t bucket = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (bucket >= nb) return;  // no block-wide barrier below
  const int64_t base = bucket * d;
  const int nj = (int)((n - base) < d ? (n - base) : d);
  const int kk = nj < K ? nj : K;
  float* row = row_all[wave];
  // whole buckets (nj = d, a multiple of 4) clear and read the row with
  // 128-bit LDS accesses and store the output nontemporally, as the other
  // dequantizers do
  const bool whole = nj == d;
  if (whole) {
    for (int i = 4 * lane; i < nj; i += 256)
      *reinterpret_cast<float4*>(row + i) = make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    for (int i = lane; i < nj; i += 64) row[i] = 0.f;
  }
  const int fw = ib + BITS;
  const uint32_t imask = (1u << ib) - 1u;
  for (int w = 0; w < W; ++w) {
    const uint32_t* recw = reinterpret_cast<const uint32_t*>(pp.codes[w]) + bucket * (int64_t)R;
    const float delta = pp.meta[w][bucket] / (float)s;
    for (int t = lane; t < kk; t += 64) {
      const int bit0 = t * fw;
      const int w0 = bit0 >> 5;
      uint64_t x = recw[w0];
      if (w0 + 1 < R) x |= (uint64_t)recw[w0 + 1] << 32;
      const uint32_t field = (uint32_t)(x >> (bit0 & 31));
      const uint32_t idx = field & imask;
      const uint32_t u = (field >> ib) & ((1u << BITS) - 1u);
      const uint32_t m = 1u << (BITS - 1);
      const int c = (int)((u ^ m) - m);
      if ((int)idx < nj) row[idx] = row[idx] + (float)c * delta;
    }
  }
  for (int i = 4 * lane; i < nj; i += 256) {
    float4 a = whole ? *reinterpret_cast<const float4*>(row + i)
                     : make_float4(row[i], i + 1 < nj ? row[i + 1] : 0.f,
                                   i + 2 < nj ? row[i + 2] : 0.f,
                                   i + 3 < nj ? row[i + 3] : 0.f);
    float4 rr = make_float4(alpha * a.x, alpha * a.y, alpha * a.z, alpha * a.w);
    if (beta != 0.f) {
      const float4 old = load4(out, base + i, base + nj);
      rr.x = rr.x + beta * old.x;
      rr.y = rr.y + beta * old.y;
      rr.z = rr.z + beta * old.z;
      rr.w = rr.w + beta * old.w;
    }
    if (whole) store4_nt(out + base + i, rr);
    else store4(out, base + i, base + nj, rr);
  }
}

}  // namespace

int topk_record_words(int d, int bits, int K) {
  const int ib = __builtin_ctz((unsigned)d);
  return (int)(((int64_t)K * (ib + bits) + 31) / 32);
}

int launch_topk_quant(const LaunchDesc& L, int64_t n, const float* g, float* e,
                      uint64_t seed, uint32_t step, uint8_t* codes,
                      float* meta, hipStream_t st) {
  const int64_t nb = (n + L.d - 1) / L.d;
  const int ib = __builtin_ctz((unsigned)L.d);
  const int R = topk_record_words(L.d, L.bits, L.L);
  const int nearest = (L.flags & GQ_FLAG_NEAREST) ? 1 : 0;
  const dim3 grid((uint32_t)((nb + kWavesPerBlock - 1) / kWavesPerBlock));
  const dim3 block(64 * kWavesPerBlock);
#define GQ_TQ(BITS, V)                                                         \
  hipLaunchKernelGGL((k_topk_quant<BITS, V>), grid, block, 0, st, n, nb, L.d,  \
                     ib, L.L, R, g, e, (uint32_t)seed, (uint32_t)(seed >> 32), \
                     step, L.s, nearest, codes, meta)
#define GQ_TQ_V(BITS)            \
  if (L.d <= 256) GQ_TQ(BITS, 1); \
  else GQ_TQ(BITS, 2);
  switch (L.bits) {
    case 2: GQ_TQ_V(2) break;
    case 3: GQ_TQ_V(3) break;
    case 4: GQ_TQ_V(4) break;
    case 8: GQ_TQ_V(8) break;
    default: return (int)hipErrorInvalidValue;
  }
#undef GQ_TQ_V
#undef GQ_TQ
  return (int)hipGetLastError();
}

int launch_topk_deq(const LaunchDesc& L, int64_t n, int W, const PayloadPtrs& pp,
                    float alpha, float beta, float* out, hipStream_t st) {
  const int64_t nb = (n + L.d - 1) / L.d;
  const int ib = __builtin_ctz((unsigned)L.d);
  const int R = topk_record_words(L.d, L.bits, L.L);
  const dim3 grid((uint32_t)((nb + kWavesPerBlock - 1) / kWavesPerBlock));
  const dim3 block(64 * kWavesPerBlock);
#define GQ_TD(BITS)                                                          \
  hipLaunchKernelGGL((k_topk_deq<BITS>), grid, block, 0, st, n, nb, L.d, ib, \
                     L.L, R, L.s, W, pp, alpha, beta, out)
  switch (L.bits) {
    case 2: GQ_TD(2); break;
    case 3: GQ_TD(3); break;
    case 4: GQ_TD(4); break;
    case 8: GQ_TD(8); break;
    default: return (int)hipErrorInvalidValue;
  }
#undef GQ_TD
  return (int)hipGetLastError();
}

}  // namespace gq
