// stream_quant.hip — one-pass quantizers whose per-bucket levels come from a
// reduction: max-abs uniform (QSGD / ternary / INT8), the sign split, and
// two levels at the bucket's minimum and maximum with random rounding
// (ORQ with L = 2 and no clipping: the levels of the greedy before any
// insertion, read as BinGrad-pb).
//
// One HBM pass per bucket: 128-bit loads of g (and e), p = g + e kept in
// registers, a group reduction for the bucket's levels, then Philox rounding,
// packing and the residual store, all from registers.
//
// Work mapping (d = 4 * G * V):  a group of G lanes owns one bucket; lane t
// holds the float4s t, t+G, ..., t+(V-1)G of it, so every load instruction
// of the group reads G consecutive 16-byte vectors.  G <= 64 groups live
// inside one wave (256-thread blocks hold 256/G buckets); G > 64 spans G/64
// waves of one block and reduces through LDS.
#include <type_traits>

#include "common.hpp"

namespace gq {
namespace {

template <int G>
struct BlockCfg {
  static constexpr int kThreads = G <= 64 ? 256 : G;
  static constexpr int kGroups = kThreads / G;
  static constexpr int kWaves = kThreads / 64;
};

// Reduce across the G/64 waves of a bucket (G > 64) through LDS.
template <int G>
__device__ __forceinline__ float bucket_max(float v, float* red) {
  if constexpr (G <= 64) {
    return group_max<G>(v);
  } else {
    v = group_max<64>(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < G / 64; ++w) m = fmaxf(m, red[w]);
    return m;
  }
}

// Two maxima over the bucket with one barrier (G > 64).
template <int G>
__device__ __forceinline__ void bucket_max2(float& a, float& b, float* red) {
  if constexpr (G <= 64) {
    a = group_max<G>(a);
    b = group_max<G>(b);
  } else {
    a = group_max<64>(a);
    b = group_max<64>(b);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
      red[2 * wave + 0] = a;
      red[2 * wave + 1] = b;
    }
    __syncthreads();
    a = red[0];
    b = red[1];
#pragma unroll
    for (int w = 1; w < G / 64; ++w) {
      a = fmaxf(a, red[2 * w + 0]);
      b = fmaxf(b, red[2 * w + 1]);
    }
  }
}

// Side sums and counts of the sign split over the bucket.  Each side's
// values share a sign, so plain fp64 sums have no cancellation: relative
// error below d * 2^-53 (< 4e-12 at d = 32768), far inside what rounding the
// means to fp32 can see in all but a vanishing fraction of buckets.
template <int G>
__device__ __forceinline__ void bucket_side_sums(double& sn, double& sp, int& nn,
                                                 int& np, double* redd,
                                                 int* redi) {
  constexpr int GW = G <= 64 ? G : 64;
  auto addd = [](double a, double b) { return a + b; };
  auto addi = [](int a, int b) { return a + b; };
  sn = group_reduce<GW>(sn, addd);
  sp = group_reduce<GW>(sp, addd);
  nn = group_reduce<GW>(nn, addi);
  np = group_reduce<GW>(np, addi);
  if constexpr (G > 64) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int NW = G / 64;
    if (lane == 0) {
      redd[2 * wave + 0] = sn;
      redd[2 * wave + 1] = sp;
      redi[2 * wave + 0] = nn;
      redi[2 * wave + 1] = np;
    }
    __syncthreads();
    sn = redd[0];
    sp = redd[1];
    nn = redi[0];
    np = redi[1];
    // sequential over the waves: unrolling would hoist every partial into
    // registers at once
#pragma unroll 1
    for (int w = 1; w < NW; ++w) {
      sn += redd[2 * w + 0];
      sp += redd[2 * w + 1];
      nn += redi[2 * w + 0];
      np += redi[2 * w + 1];
    }
  }
}

// BITS = 0 selects dense packing (uniform scheme, A = 2s+1 <= 15 symbols):
// see store_dense_chunk.  Every wave then holds aligned 256-element chunks
// (per v, the wave's 64 lanes cover 256 consecutive elements), and groups
// past the last bucket stay to the end: all their loads and stores are
// bounds-checked, and the field assembly needs all 64 lanes.
// CHUNKED (1024 lanes of 8 float4s, d = 32768; the min/max and the packed
// uniform quantizers): at most 64 VGPRs, so that two buckets share a CU and
// one's reduction barrier overlaps the other's loads and stores (one bucket
// per CU left the CU without memory traffic while its waves met).  The
// float4s are loaded in two halves, the first summed before the second is
// issued, and the random words are drawn per float4 in the coding pass
// instead of during the loads.  (The sign split's fp64 side sums and the
// dense packing do not fit 64 VGPRs without spilling.)
template <int SCHEME, int BITS, int G, int V>
constexpr bool stream_chunked() {
  return G == 1024 && V == 8 && (SCHEME == ORQ || (SCHEME == UNIFORM && BITS != 0));
}

template <int SCHEME, int BITS, int G, int V>
__global__ __launch_bounds__(BlockCfg<G>::kThreads, (stream_chunked<SCHEME, BITS, G, V>() ? 8 : 1))
void k_stream_quant(
    int64_t n, int64_t nb, const float* __restrict__ g, float* __restrict__ e,
    uint32_t k0, uint32_t k1, uint32_t step, int s, int nearest,
    uint8_t* __restrict__ codes, float* __restrict__ meta, int64_t code_bytes,
    uint32_t A4, int W) {
  constexpr int D = 4 * G * V;
  constexpr bool DENSE = BITS == 0;
  constexpr bool RANDOM = SCHEME == UNIFORM || SCHEME == ORQ;  // Philox draws
  constexpr int NW = G > 64 ? G / 64 : 1;
  __shared__ float red_f[NW];
  __shared__ float red_f2[2 * NW];
  __shared__ double red_d[2 * NW];
  __shared__ int red_i[2 * NW];

  const int lane = threadIdx.x % G;
  const int64_t bucket =
      (int64_t)blockIdx.x * BlockCfg<G>::kGroups + threadIdx.x / G;
  if (!DENSE && bucket >= nb) return;  // whole groups leave together
  const int64_t base = bucket * D;

  // ---- load p = g (+ e) ------------------------------------------------
  // Random words for the uniform scheme, or (nearest) words whose u is
  // exactly 1/2, so that a value rounds up iff q > 1/2.  They depend on the
  // element index only and are drawn while the loads are in flight.
  constexpr bool CHUNKED = stream_chunked<SCHEME, BITS, G, V>();
  auto word4 = [&](int v) {
    uint4 w = make_uint4(kHalfWord, kHalfWord, kHalfWord, kHalfWord);
    if (!nearest && codes != nullptr) {
      const uint64_t ctr = (uint64_t)(base + 4 * (lane + G * v)) >> 2;
      w = philox4x32_10(k0, k1, (uint32_t)ctr, (uint32_t)(ctr >> 32), step, 0u);
    }
    return w;
  };
  uint4 wr[RANDOM && !CHUNKED ? V : 1];
  auto draw = [&]() {
    if constexpr (RANDOM && !CHUNKED) {
#pragma unroll
      for (int v = 0; v < V; ++v) wr[v] = word4(v);
    }
  };
  auto words = [&](int v) {
    if constexpr (CHUNKED) return word4(v);
    else return wr[RANDOM ? v : 0];
  };
  float4 p[V], r[V];
  auto add_residual = [&]() {
    if (e != nullptr) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        p[v].x = p[v].x + r[v].x;
        p[v].y = p[v].y + r[v].y;
        p[v].z = p[v].z + r[v].z;
        p[v].w = p[v].w + r[v].w;
      }
    }
  };
  // A bucket wholly inside the gradient (every bucket but possibly the
  // last; the test is uniform over the group) loads with 128-bit
  // nontemporal loads, all issued before any use; the last bucket checks
  // each element.
  const bool whole = base + D <= n;
  // elements of the bucket inside the gradient (0 for groups past the end)
  const int rem = (int)(n - base < D ? (n - base > 0 ? n - base : 0) : D);
  if (whole && CHUNKED) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // (the second half's loads stay behind the first half's sums)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int v = h * (V / 2); v < (h + 1) * (V / 2); ++v)
        p[v] = load4_nt(g + base + 4 * (lane + G * v));
      if (e != nullptr) {
#pragma unroll
        for (int v = h * (V / 2); v < (h + 1) * (V / 2); ++v) {
          const float4 rv = load4_nt(e + base + 4 * (lane + G * v));
          p[v].x = p[v].x + rv.x;
          p[v].y = p[v].y + rv.y;
          p[v].z = p[v].z + rv.z;
          p[v].w = p[v].w + rv.w;
        }
      }
    }
  } else if (whole) {
#pragma unroll
    for (int v = 0; v < V; ++v)
      p[v] = load4_nt(g + base + 4 * (lane + G * v));
    if (e != nullptr) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        r[v] = load4_nt(e + base + 4 * (lane + G * v));
    }
    draw();
    add_residual();
  } else if (CHUNKED) {
    // (32-bit offsets from the bucket's base: no 64-bit index per float4)
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int off = 4 * (lane + G * v);
      p[v] = load4(g + base, off, rem);
      if (e != nullptr) {
        const float4 rv = load4(e + base, off, rem);
        p[v].x = p[v].x + rv.x;
        p[v].y = p[v].y + rv.y;
        p[v].z = p[v].z + rv.z;
        p[v].w = p[v].w + rv.w;
      }
    }
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int64_t i = base + 4 * (lane + G * v);
      p[v] = load4(g, i, n);
      if (e != nullptr) r[v] = load4(e, i, n);
    }
    draw();
    add_residual();
  }

  // The rest, with the elements of each float4 that lie in the gradient
  // known to be all four where WH (CHUNKED whole buckets: one bucket per
  // block, so every thread of the block takes the same instance; elsewhere
  // groups of one wave may differ, and the dense packing exchanges lanes).
  auto finish = [&](auto wh_tag) {
  constexpr bool WH = decltype(wh_tag)::value;
  auto nreal_of = [&](int v) -> int {
    if constexpr (WH) {
      return 4;
    } else {
      const int left = rem - 4 * (lane + G * v);
      return left >= 4 ? 4 : (left > 0 ? left : 0);
    }
  };
  // ---- per-bucket levels ----------------------------------------------
  // UNIFORM: M = max |p| (absent tail elements load as 0, which never
  // raises a max-abs).  ORQ (L = 2): minimum and maximum over the real
  // elements.  BIN_SIGN: side means over the real elements.
  float lvl0 = 0.f, lvl1 = 0.f;
  if constexpr (SCHEME == UNIFORM) {
    float m = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(p[v].x), fabsf(p[v].y)),
                         fmaxf(fabsf(p[v].z), fabsf(p[v].w))));
    lvl0 = bucket_max<G>(m, red_f);
  } else if constexpr (SCHEME == ORQ) {
    float hi = -INFINITY, nlo = -INFINITY;  // max p and max (-p)
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int nreal = nreal_of(v);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x = comp(p[v], k);
        hi = k < nreal ? fmaxf(hi, x) : hi;
        nlo = k < nreal ? fmaxf(nlo, -x) : nlo;
      }
    }
    bucket_max2<G>(hi, nlo, red_f2);
    lvl1 = hi;
    lvl0 = -nlo;
    // a zero level is +0 (levels are values of the sorted bucket, in which
    // -0 and +0 are one value)
    lvl0 = lvl0 == 0.f ? 0.f : lvl0;
    lvl1 = lvl1 == 0.f ? 0.f : lvl1;
  } else {
    // Each lane sums its own values of one sign in plain fp64, then the
    // lanes' sums are added up the same way.
    double sn = 0.0, sp = 0.0;
    int nn = 0, np = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int nreal = nreal_of(v);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x = comp(p[v], k);
        const bool real = k < nreal;
        const bool up = x >= 0.f;
        sp += (real && up) ? (double)x : 0.0;
        sn += (real && !up) ? (double)x : 0.0;
        np += (real && up) ? 1 : 0;
        nn += (real && !up) ? 1 : 0;
      }
    }
    bucket_side_sums<G>(sn, sp, nn, np, red_d, red_i);
    lvl0 = nn ? (float)(sn / (double)nn) : 0.f;
    lvl1 = np ? (float)(sp / (double)np) : 0.f;
  }

  if (lane == 0 && bucket < nb) {
    if constexpr (SCHEME == UNIFORM) {
      meta[bucket] = lvl0;
    } else {
      meta[2 * bucket + 0] = lvl0;
      meta[2 * bucket + 1] = lvl1;
    }
  }
  if (codes == nullptr) return;  // levels only

  // ---- round, pack, residual ---------------------------------------------
  const float M = lvl0;
  const float sf = (float)s;
  // A bucket whose max-abs is below 2^-96 is scaled by 2^96 first (exact)
  // so that s / M stays finite; for all other buckets the factor is 1.
  const float up = M < 0x1p-96f ? 0x1p96f : 1.0f;
  const float inv = M > 0.f ? sf / (M * up) : 0.f;
  const float delta = M / sf;

  // The rounding pass, specialised on whether the bucket is scaled (the
  // factor 1 multiplies exactly, so the common case skips it).
  auto code_pass = [&](auto scaled_tag) {
    constexpr bool SCALED = decltype(scaled_tag)::value;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int64_t i = base + 4 * (lane + G * v);
      uint32_t c[4];
      int sc[4] = {0, 0, 0, 0};  // signed codes (dense digits are sc + s)
      float4 xh;
      if constexpr (SCHEME == UNIFORM) {
        const uint4 wv = words(v);
        const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int ci = uniform_code<SCALED>(comp(p[v], k), up, inv, sf, ws[k]);
          sc[k] = ci;
          c[k] = DENSE ? 0u : ((uint32_t)ci & ((1u << BITS) - 1u));
          const float xk = (float)ci * delta;
          if (k == 0) xh.x = xk;
          if (k == 1) xh.y = xk;
          if (k == 2) xh.z = xk;
          if (k == 3) xh.w = xk;
        }
      } else if constexpr (SCHEME == ORQ) {
        // q = (p - a) / (b - a) in fp32; up iff u < q (nearest: q > 1/2); a
        // value equal to a level takes it (the lower one when a = b)
        const uint4 wv = words(v);
        const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
        const float den = lvl1 - lvl0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x = comp(p[v], k);
          const float q = (x - lvl0) / den;
          c[k] = x == lvl0 ? 0u : (x == lvl1 || u24(ws[k]) < q ? 1u : 0u);
          const float xk = c[k] ? lvl1 : lvl0;
          if (k == 0) xh.x = xk;
          if (k == 1) xh.y = xk;
          if (k == 2) xh.z = xk;
          if (k == 3) xh.w = xk;
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x = comp(p[v], k);
          c[k] = x >= 0.f ? 1u : 0u;
          const float xk = c[k] ? lvl1 : lvl0;
          if (k == 0) xh.x = xk;
          if (k == 1) xh.y = xk;
          if (k == 2) xh.z = xk;
          if (k == 3) xh.w = xk;
        }
      }
      // absent tail elements pack as 0
      const int nreal = nreal_of(v);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k >= nreal) c[k] = 0u;
      if constexpr (DENSE) {
        const uint32_t A = 2u * (uint32_t)s + 1u;
        uint32_t u = 0u;
#pragma unroll
        for (int k = 3; k >= 0; --k)
          u = __umul24(u, A) + (k < nreal ? (uint32_t)(sc[k] + s) : 0u);
        store_dense_chunk(codes, i - 4 * (threadIdx.x & 63), u, A4, W, code_bytes);
      } else {
        store_field<BITS, G>(codes, i, lane, field4<BITS>(c[0], c[1], c[2], c[3]),
                             code_bytes);
      }
      if (e != nullptr && (WH || i < n)) {
        float4 r;
        r.x = p[v].x - xh.x;
        r.y = p[v].y - xh.y;
        r.z = p[v].z - xh.z;
        r.w = p[v].w - xh.w;
        if (WH || whole) store4_nt(e + i, r);
        else store4(e, i, n, r);
      }
    }
  };
  if (up == 1.0f) code_pass(std::false_type{});
  else code_pass(std::true_type{});
  };
  if (CHUNKED && whole) finish(std::true_type{});
  else finish(std::false_type{});
}

template <int SCHEME, int BITS, int G, int V>
int launch_one(int64_t n, const float* g, float* e, uint64_t seed,
               uint32_t step, int s, int nearest, uint8_t* codes, float* meta,
               int64_t code_bytes, uint32_t A4, int W, hipStream_t st) {
  constexpr int D = 4 * G * V;
  const int64_t nb = (n + D - 1) / D;
  const int64_t blocks = (nb + BlockCfg<G>::kGroups - 1) / BlockCfg<G>::kGroups;
  hipLaunchKernelGGL((k_stream_quant<SCHEME, BITS, G, V>), dim3((uint32_t)blocks),
                     dim3(BlockCfg<G>::kThreads), 0, st, n, nb, g, e,
                     (uint32_t)seed, (uint32_t)(seed >> 32), step, s, nearest,
                     codes, meta, code_bytes, A4, W);
  return (int)hipGetLastError();
}

template <int SCHEME, int BITS>
int dispatch_d(int d, int64_t n, const float* g, float* e, uint64_t seed,
               uint32_t step, int s, int nearest, uint8_t* codes, float* meta,
               int64_t code_bytes, uint32_t A4, int W, hipStream_t st) {
#define GQ_CASE(D_, G_, V_)                                                  \
  case D_:                                                                   \
    return launch_one<SCHEME, BITS, G_, V_>(n, g, e, seed, step, s, nearest, \
                                            codes, meta, code_bytes, A4, W,  \
                                            st);
  // (G, V) per d, measured on 256M elements with error feedback (sign
  // split, min/max, uniform): above d = 1024 more lanes with fewer float4s
  // each beat one wave holding 8 per lane (d = 2048: 550 -> 506 us; 8192:
  // 540 -> 485 us); d = 1024 keeps one wave (4 waves: 71 % against 79 % for
  // the sign split)
  // 8-bit codes at d = 512: two waves of one float4 per lane (INT8 + EF on
  // 256M: 572 -> 556 us; the 2-bit headline is 1 % slower that way)
  if constexpr (BITS == 8) {
    if (d == 512)
      return launch_one<SCHEME, BITS, 128, 1>(n, g, e, seed, step, s, nearest,
                                              codes, meta, code_bytes, A4, W, st);
  }
  switch (d) {
    GQ_CASE(64, 16, 1)
    GQ_CASE(128, 32, 1)
    GQ_CASE(256, 64, 1)
    GQ_CASE(512, 64, 2)
    GQ_CASE(1024, 64, 4)
    GQ_CASE(2048, 256, 2)
    GQ_CASE(4096, 512, 2)
    GQ_CASE(8192, 1024, 2)
    GQ_CASE(16384, 1024, 4)
    GQ_CASE(32768, 1024, 8)
    default:
      return (int)hipErrorInvalidValue;
  }
#undef GQ_CASE
}

}  // namespace

int launch_stream_quant(const LaunchDesc& L, int64_t n, const float* g,
                        float* e, uint64_t seed, uint32_t step, uint8_t* codes,
                        float* meta, int64_t code_bytes, hipStream_t st) {
#define GQ_D(SCHEME, BITS)                                                    \
  dispatch_d<SCHEME, BITS>(L.d, n, g, e, seed, step, L.s,                     \
                           (L.flags & GQ_FLAG_NEAREST) ? 1 : 0, codes, meta,  \
                           code_bytes, L.A4, L.W, st)
  if (L.scheme == BIN_SIGN) return GQ_D(BIN_SIGN, 1);
  if (L.scheme == ORQ) return GQ_D(ORQ, 1);  // L = 2, no clipping
  if (L.dense) return GQ_D(UNIFORM, 0);
  switch (L.bits) {
    case 2:
      return GQ_D(UNIFORM, 2);
    case 3:
      return GQ_D(UNIFORM, 3);
    case 4:
      return GQ_D(UNIFORM, 4);
    case 8:
      return GQ_D(UNIFORM, 8);
    default:
      return (int)hipErrorInvalidValue;
  }
#undef GQ_D
}

}  // namespace gq
