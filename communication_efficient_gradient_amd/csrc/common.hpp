// common.hpp — device helpers shared by libgq's kernels (gfx950, wave64).
//
// Philox4x32-10, group reductions over 16..64 lanes (DPP/bpermute via
// DPP and lane swaps) and across waves (LDS), fp64 TwoSum accumulation, and the
// OR-combine that turns per-lane code fields into LSB-first stream words.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gq.h"

namespace gq {

enum Scheme { UNIFORM = 0, BIN_SIGN = 1, BIN_OPT = 2, ORQ = 3, TOPK = 4 };

constexpr int kMaxPayloads = 16;

// --------------------------------------------------------------- Philox --
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// 4x32 S-box, multipliers 0xD2511F53 / 0xCD9E8D57, key bumped by the Weyl
// constants 0x9E3779B9 / 0xBB67AE85 after each round.  Key = seed,
// counter = (i/4 lo, i/4 hi, step, 0): the four output words serve elements
// 4c .. 4c+3.  The pages ask only for rounding that is random and unbiased
// ("Gradient Quantization" glossary, Stochastic Quantization bullet); a
// counter-based generator makes the draw for element i a pure function of
// (seed, i, step), independent of the launch shape.
__device__ __forceinline__ uint4 philox4x32_10(uint32_t k0, uint32_t k1,
                                               uint32_t c0, uint32_t c1,
                                               uint32_t c2, uint32_t c3) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t m0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t m1 = (uint64_t)0xCD9E8D57u * c2;
    // three-input XORs: one gfx950 v_bitop3_b32 each (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(m1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(m0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)m1;
    c3 = (uint32_t)m0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return make_uint4(c0, c1, c2, c3);
}

// Uniform in [0, 1) from the top 24 bits of a word (exact in binary32).
__device__ __forceinline__ float u24(uint32_t w) {
  return (float)(w >> 8) * 0x1p-24f;
}

// A word whose u is exactly 1/2 (deterministic rounding to the nearest level:
// up iff q > 1/2).
constexpr uint32_t kHalfWord = 0x80000000u;

// Signed code of x on the uniform grid of a bucket with max-abs M and s
// levels per sign ("Gradient Quantization" glossary: max-abs scaling, the
// Stochastic Quantization bullet): r = min(|x| * inv, s) with inv = s / M,
// l = floor(r), q = r - l (exact), magnitude l + [u < q], u from word w.  A
// bucket with M < 2^-96 is scaled by up = 2^96 first (inv = s / (M * up));
// SCALED = false is the common case up = 1, whose multiply is exact and
// skipped.
template <bool SCALED>
__device__ __forceinline__ int uniform_code(float x, float up, float inv,
                                            float sf, uint32_t w) {
  const float ax = SCALED ? fabsf(x) * up : fabsf(x);
  const float r = fminf(ax * inv, sf);
  const float l = floorf(r);
  const float q = r - l;
  const int mag = (int)l + (u24(w) < q ? 1 : 0);
  return x < 0.f ? -mag : mag;
}

// Per-layer constants of the uniform rounding: scale-up factor, s / (M up)
// and the step M / s.
struct LayerScale {
  float up, inv, delta;
};

__device__ __forceinline__ LayerScale layer_scale(float M, float sf) {
  LayerScale c;
  c.up = M < 0x1p-96f ? 0x1p96f : 1.0f;
  c.inv = M > 0.f ? sf / (M * c.up) : 0.f;
  c.delta = M / sf;
  return c;
}

// ------------------------------------------------------- lane exchange --
// Value of lane (lane ^ o) for o = 1, 2, 4, .., 32 and for the mirror masks
// 3, 7, 15, 31, 63, without the LDS crossbar: DPP quad permutes for 1, 2
// and 3 (quad reversal), the half-row mirror for 7, the row mirror for 15,
// a quad reversal then a half-row mirror for 4 (l ^ 3 ^ 7), a row rotation
// by 8 for 8, and gfx950's row / half-wave swaps for 16 and 32 (each lane
// then picks the half that came from its partner); 31 and 63 compose a
// mirror with the swaps.  o must be a compile-time constant after
// unrolling; other values fall back to __shfl_xor.
__device__ __forceinline__ uint32_t xshfl(uint32_t v, int o);

__device__ __forceinline__ uint32_t xshfl_swap16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (threadIdx.x & 16) ? (uint32_t)r[0] : (uint32_t)r[1];
}

__device__ __forceinline__ uint32_t xshfl_swap32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & 32) ? (uint32_t)r[0] : (uint32_t)r[1];
}

__device__ __forceinline__ uint32_t xshfl(uint32_t v, int o) {
  switch (o) {
    case 3:
      return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x1B, 0xF, 0xF, false);
    case 7:
      return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);
    case 15:
      return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);
    case 31:
      return xshfl_swap16(
          (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));
    case 63:
      return xshfl_swap32(xshfl_swap16(
          (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false)));
    case 1:
      return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
    case 2:
      return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
    case 4:
      return (uint32_t)__builtin_amdgcn_mov_dpp(
          __builtin_amdgcn_mov_dpp((int)v, 0x1B, 0xF, 0xF, false), 0x141, 0xF,
          0xF, false);
    case 8:
      return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);
    case 16:
      return xshfl_swap16(v);
    case 32:
      return xshfl_swap32(v);
    default:
      return (uint32_t)__shfl_xor((int)v, o, 64);
  }
}

__device__ __forceinline__ float xshfl(float v, int o) {
  return __uint_as_float(xshfl(__float_as_uint(v), o));
}

__device__ __forceinline__ int xshfl(int v, int o) {
  return (int)xshfl((uint32_t)v, o);
}

__device__ __forceinline__ double xshfl(double v, int o) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = xshfl((uint32_t)b, o), hi = xshfl((uint32_t)(b >> 32), o);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// The value of lane (lane ^ M) through the LDS crossbar: ds_swizzle inside
// 32-lane halves (bit-mask mode: and 0x1f, xor M), ds_bpermute across them.
// No VALU instruction for the exchange itself, so a VALU-bound kernel with
// several independent exchanges in flight leaves them to the LDS pipe (a
// single dependent exchange is faster with xshfl's DPP moves).  Workgroups
// are whole waves, so threadIdx.x & 63 is the lane.
template <int M>
__device__ __forceinline__ float lane_xor_ds(float v) {
  static_assert(M > 0 && M < 64, "lane mask");
  if constexpr (M < 32) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1f | (M << 10)));
  } else {
    const int src = (int)((threadIdx.x & 63u) ^ (unsigned)M) << 2;
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(v)));
  }
}

// ------------------------------------------------------- group reductions --
// Butterfly reductions over aligned groups of G lanes inside one wave
// (G <= 64): exchange distances G/2, G/4, ..., 1, unrolled at compile time.
template <int G, typename V, typename Op>
__device__ __forceinline__ V group_reduce(V v, Op op) {
  if constexpr (G > 1) {
    v = op(v, xshfl(v, G / 2));
    return group_reduce<G / 2>(v, op);
  } else {
    return v;
  }
}

template <int G>
__device__ __forceinline__ float group_max(float v) {
  return group_reduce<G>(v, [](float a, float b) { return fmaxf(a, b); });
}

template <int G>
__device__ __forceinline__ int group_sum_i(int v) {
  return group_reduce<G>(v, [](int a, int b) { return a + b; });
}

template <int K>
__device__ __forceinline__ uint32_t group_or(uint32_t v) {
  return group_reduce<K>(v, [](uint32_t a, uint32_t b) { return a | b; });
}

// fp64 sum with a running error term (Knuth TwoSum, branch-free).  The
// result s + c is the exact sum up to O(n u^2) relative error, so means
// rounded to fp32 agree with any other near-exact summation order.
struct Sum2 {
  double s, c;
};

__device__ __forceinline__ void two_sum_add(Sum2& a, double x) {
  const double t = a.s + x;
  const double bp = t - a.s;
  const double err = (a.s - (t - bp)) + (x - bp);
  a.s = t;
  a.c += err;
}

__device__ __forceinline__ Sum2 two_sum_merge(Sum2 a, Sum2 b) {
  Sum2 r = a;
  two_sum_add(r, b.s);
  r.c += b.c;
  return r;
}

template <int G>
__device__ __forceinline__ Sum2 group_sum2(Sum2 v) {
  if constexpr (G > 1) {
    Sum2 w;
    w.s = xshfl(v.s, G / 2);
    w.c = xshfl(v.c, G / 2);
    return group_sum2<G / 2>(two_sum_merge(v, w));
  } else {
    return v;
  }
}

// ------------------------------------------------------------- packing --
// Pack four codes of BITS bits (already masked) into one 4*BITS-bit field,
// element 0 in the lowest bits.
template <int BITS>
__device__ __forceinline__ uint32_t field4(uint32_t c0, uint32_t c1,
                                           uint32_t c2, uint32_t c3) {
  return c0 | (c1 << BITS) | (c2 << (2 * BITS)) | (c3 << (3 * BITS));
}

// Load the float4 at element index i (a multiple of 4) with a guarded tail.
__device__ __forceinline__ float4 load4(const float* __restrict__ a, int64_t i,
                                        int64_t n) {
  if (i + 3 < n) return *reinterpret_cast<const float4*>(a + i);
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  if (i + 0 < n) r.x = a[i + 0];
  if (i + 1 < n) r.y = a[i + 1];
  if (i + 2 < n) r.z = a[i + 2];
  return r;
}

__device__ __forceinline__ void store4(float* __restrict__ a, int64_t i,
                                       int64_t n, float4 v) {
  if (i + 3 < n) {
    *reinterpret_cast<float4*>(a + i) = v;
    return;
  }
  if (i + 0 < n) a[i + 0] = v.x;
  if (i + 1 < n) a[i + 1] = v.y;
  if (i + 2 < n) a[i + 2] = v.z;
}

// 128-bit loads and stores with the nontemporal hint, for streams that are
// touched once per launch (the gradient, the residual, the aggregate):
// measured faster than cached accesses once the stream exceeds the
// last-level cache.  `p` must be 16-byte aligned.
typedef float nt_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load4_nt(const float* p) {
  const nt_f4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store4_nt(float* p, float4 r) {
  const nt_f4 v = {r.x, r.y, r.z, r.w};
  __builtin_nontemporal_store(v, reinterpret_cast<nt_f4*>(p));
}

__device__ __forceinline__ float comp(const float4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// Store this lane's 4*BITS-bit field into the LSB-first stream.  The field
// of lane t covers elements idx .. idx+3; K consecutive lanes together fill
// whole 32-bit words (K = 8/BITS), or three words for BITS = 3.  Words that
// start at or past code_bytes are skipped (the buffer holds code_bytes
// rounded up to 16).
template <int BITS, int G>
__device__ __forceinline__ void store_field(uint8_t* __restrict__ codes,
                                            int64_t idx, int lane,
                                            uint32_t field,
                                            int64_t code_bytes) {
  if constexpr (BITS == 3) {
    const int q = lane & 7;
    const int off = 12 * q;
    const uint64_t x = (uint64_t)field << (off & 31);
    const int wi = off >> 5;
    uint32_t w0 = wi == 0 ? (uint32_t)x : 0u;
    uint32_t w1 = wi == 1 ? (uint32_t)x : (wi == 0 ? (uint32_t)(x >> 32) : 0u);
    uint32_t w2 = wi == 2 ? (uint32_t)x : (wi == 1 ? (uint32_t)(x >> 32) : 0u);
    w0 = group_or<8>(w0);
    w1 = group_or<8>(w1);
    w2 = group_or<8>(w2);
    if (q < 3) {
      const int64_t byte = ((idx - 4 * q) >> 5) * 12 + 4 * q;
      if (byte < code_bytes) {
        const uint32_t w = q == 0 ? w0 : (q == 1 ? w1 : w2);
        *reinterpret_cast<uint32_t*>(codes + byte) = w;
      }
    }
  } else {
    constexpr int K = 8 / BITS;
    const int q = lane & (K - 1);
    uint32_t w = field << (4 * BITS * q);
    w = group_or<K>(w);
    if (q == 0) {
      const int64_t byte = (idx * BITS) >> 3;
      if (byte < code_bytes) *reinterpret_cast<uint32_t*>(codes + byte) = w;
    }
  }
}

// Store the codes of VEC consecutive elements (idx .. idx+VEC-1, idx a
// multiple of VEC) held by this lane as one VEC*BITS-bit field, element idx
// in the lowest bits.  The lanes of a wave must hold consecutive VEC-element
// chunks (lane t chunk c0 + t): K = 32/(VEC*BITS) neighbouring lanes OR their
// fields into one 32-bit stream word, and for BITS = 3 the 32/VEC lanes that
// cover 32 elements build three words.  Words that start at or past
// code_bytes are skipped (the buffer holds code_bytes rounded up to 16).
template <int BITS, int VEC>
__device__ __forceinline__ void store_chunk(uint8_t* __restrict__ codes,
                                            int64_t idx, int lane,
                                            uint32_t field, int64_t code_bytes) {
  constexpr int FB = VEC * BITS;
  if constexpr (BITS == 3) {
    constexpr int Q = 32 / VEC;
    const int q = lane & (Q - 1);
    const int off = FB * q;
    const uint64_t x = (uint64_t)field << (off & 31);
    const int wi = off >> 5;
    uint32_t w0 = wi == 0 ? (uint32_t)x : 0u;
    uint32_t w1 = wi == 1 ? (uint32_t)x : (wi == 0 ? (uint32_t)(x >> 32) : 0u);
    uint32_t w2 = wi == 2 ? (uint32_t)x : (wi == 1 ? (uint32_t)(x >> 32) : 0u);
    w0 = group_or<Q>(w0);
    w1 = group_or<Q>(w1);
    w2 = group_or<Q>(w2);
    if (q < 3) {
      const int64_t first = idx - (int64_t)VEC * q;
      const int64_t byte = (first >> 5) * 12 + 4 * q;
      if (byte < code_bytes) {
        const uint32_t w = q == 0 ? w0 : (q == 1 ? w1 : w2);
        *reinterpret_cast<uint32_t*>(codes + byte) = w;
      }
    }
  } else {
    constexpr int K = 32 / FB;
    const int q = lane & (K - 1);
    uint32_t w = K > 1 ? field << (FB * q) : field;
    w = group_or<K>(w);
    if (q == 0) {
      const int64_t byte = (idx * BITS) >> 3;
      if (byte < code_bytes) *reinterpret_cast<uint32_t*>(codes + byte) = w;
    }
  }
}

// ------------------------------------------------------- dense packing --
// The 64 lanes of a wave hold the 256 consecutive elements chunk0 ..
// chunk0+255 (chunk0 a multiple of 256), lane l the elements chunk0 + 4l ..
// +3, given as u = d0 + A d1 + A^2 d2 + A^3 d3 (d0 for the first element).
// Lanes 2f and 2f+1 form field f = u_2f + A^4 u_2f+1 (< A^8 <= 2^32); the
// chunk's 32 fields of W bits (13 <= W <= 32) fill exactly W stream words,
// words c*W .. c*W + W-1 for chunk c, and lane L < W assembles word L from
// the (at most four) fields that overlap it.  All 64 lanes must take part.
// Words that start at or past code_bytes are skipped.
__device__ __forceinline__ void store_dense_chunk(uint8_t* __restrict__ codes,
                                                  int64_t chunk0, uint32_t u,
                                                  uint32_t A4, int W,
                                                  int64_t code_bytes) {
  const int lane = threadIdx.x & 63;
  const uint32_t V = u + A4 * xshfl(u, 1);  // meaningful on even lanes
  const int L = lane < W ? lane : 0;
  const int f0 = (32 * L) / W;
  uint32_t word = 0u;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int f = f0 + r;
    const uint32_t vf = (uint32_t)__shfl((int)V, 2 * (f < 32 ? f : 31), 64);
    const int off = W * f - 32 * L;  // bit of field f inside word L
    if (f < 32 && off < 32) word |= off >= 0 ? (vf << off) : (vf >> (-off));
  }
  if (lane < W) {
    const int64_t byte = (chunk0 >> 8) * 4 * (int64_t)W + 4 * lane;
    if (byte < code_bytes) *reinterpret_cast<uint32_t*>(codes + byte) = word;
  }
}

// Four 4-bit digits (first in the low nibble) as one base-A number,
// first digit least significant.
__device__ __forceinline__ uint32_t nibbles_to_base(uint32_t nib, uint32_t A) {
  uint32_t u = (nib >> 12) & 0xFu;
  u = __umul24(u, A) + ((nib >> 8) & 0xFu);
  u = __umul24(u, A) + ((nib >> 4) & 0xFu);
  return __umul24(u, A) + (nib & 0xFu);
}

// Digit split of a dense field without integer division.  For an integer
// v and divisor q, floor(v / q) = floor((v + 1/2) / q), and the fractional
// part of (v + 1/2) / q lies in [1/(2q), 1 - 1/(2q)].  The product
// (v + 1/2) * fl(1/q), evaluated as one fused multiply-add, is within a
// relative 2^-(p-1) of that quotient (p = 53 or 24 bits), so truncating it
// is exact whenever quotient * 2^-(p-1) < 1/(2q):
//   * fp64, v < 2^32, q = A^4 <= 2^16: error < 2^-20 against a margin of
//     at least 2^-17;
//   * fp32, v < 2^16, q = A <= 16: error < 2^-8 against at least 2^-5.
// rq = fl(1/q) and hq = rq / 2 (exact) come from the host.
__device__ __forceinline__ uint32_t div_field(uint32_t v, double rq, double hq) {
  return (uint32_t)__fma_rn((double)v, rq, hq);
}
__device__ __forceinline__ uint32_t div_digit(uint32_t v, float rq, float hq) {
  return (uint32_t)__fmaf_rn((float)v, rq, hq);
}

// Reciprocals for the digit split of a dense stream with alphabet A.
struct DenseRecip {
  double rA4, hA4;  // fl(1/A^4) and half of it
  float rA, hA;     // fl(1/A) and half of it
};

// The four digits (element 4f .. 4f+3) of float4 group f of a dense stream,
// digit k in bits 8k .. 8k+7.  Group f is the low (f even) or high (f odd)
// base-A^4 half of field f/2.  Groups whose two stream words lie inside
// code_bytes load them whole; otherwise bytes are read one by one.
__device__ __forceinline__ uint32_t load_dense4(const uint8_t* __restrict__ c,
                                                int64_t f, int W, uint32_t A,
                                                uint32_t A4,
                                                const DenseRecip& r,
                                                int64_t code_bytes) {
  const int64_t bit0 = (int64_t)W * (f >> 1);
  const int64_t wi = bit0 >> 5;
  uint64_t x;
  if (4 * wi + 8 <= code_bytes) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(c);
    x = (uint64_t)w[wi] | ((uint64_t)w[wi + 1] << 32);
  } else {
    x = 0;
    for (int b = 0; b < 8; ++b)
      if (4 * wi + b < code_bytes) x |= (uint64_t)c[4 * wi + b] << (8 * b);
  }
  uint32_t v = (uint32_t)(x >> (bit0 & 31));
  if (W < 32) v &= (1u << W) - 1u;
  const uint32_t hi = div_field(v, r.rA4, r.hA4);  // < A^4 <= 2^16
  v = (f & 1) ? hi : v - __umul24(hi, A4);
  uint32_t out = 0;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const uint32_t q = div_digit(v, r.rA, r.hA);
    out |= (v - __umul24(q, A)) << (8 * k);
    v = q;
  }
  return out | (v << 24);
}

// ---------------------------------------------------------- layers --
// Per-layer scale (TernGrad): the flat gradient is the concatenation of nl
// layers, layer l = elements [off[l], off[l+1]).  Kernels that walk it in
// tiles find the layers meeting a tile once per block.  With nl <
// kOffCache the block first copies off into LDS (one load per thread,
// issued before the tile's data loads, so the search waits for it alone);
// otherwise one wave searches off in global memory.  The layer starts
// inside the tile (at most kMaxStarts) are then kept in LDS; a tile met by
// more layers looks each element up.  Every layer index is clamped to
// [0, nl), so any contents of off give in-bounds accesses.
constexpr int kMaxStarts = 32;     // layer starts inside one tile kept in LDS
constexpr int kOffCache = 1024;    // offsets copied to LDS when nl < this
constexpr int kOffPerThread = kOffCache / 256;

// Layer holding flat element x: the largest l in [0, nl) with off[l] <= x
// (empty layers are passed over); off may be global or LDS memory.
__device__ __forceinline__ int layer_of(const int64_t* __restrict__ off,
                                        int nl, int64_t x) {
  int lo = 0, hi = nl;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= x) lo = mid;
    else hi = mid;
  }
  return lo;
}

// The same, found by the 64 lanes of one wave together in global memory
// (every lane returns it): each round reads 64 evenly spaced offsets of the
// remaining range and keeps the stretch after the last one <= x.
__device__ __forceinline__ int layer_of_wave(const int64_t* __restrict__ off,
                                             int nl, int64_t x) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = nl;  // the layer lies in [lo, hi)
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) >> 6;
    const int idx = lo + lane * step;
    const bool ok = idx < hi && off[idx] <= x;
    const uint64_t m = __ballot(ok);
    const int last = m ? 63 - __clzll((long long)m) : 0;
    lo += last * step;
    hi = lo + step < hi ? lo + step : hi;
  }
  return lo;
}

// LDS of a tile's layer search: offc = off[0..nl] when nl < kOffCache,
// otherwise starts[k] = off[lf + 1 + k] for the layers starting inside it.
struct TileLayers {
  int64_t starts[kMaxStarts];
  int64_t offc[kOffCache];
};

// Step 1 (before the tile's data loads): this thread's share of off.
__device__ __forceinline__ void prefetch_offsets(int64_t (&o)[kOffPerThread],
                                                 const int64_t* __restrict__ off,
                                                 int nl) {
#pragma unroll
  for (int j = 0; j < kOffPerThread; ++j) {
    const int idx = threadIdx.x + 256 * j;
    o[j] = (nl < kOffCache && idx <= nl) ? off[idx] : 0;
  }
}

// Step 2: the tile [t0, t1).  Blocks of 256 threads; every thread calls it
// and gets the tile's first layer lf and the number ns of layers starting
// inside it (-1 when there are more than kMaxStarts).  With off in LDS
// (nl < kOffCache) one barrier: lf and lf + ns are the counts of off[1..nl)
// at or below t0 and t1 - 1 (the largest l with off[l] <= x, empty layers
// passed over), summed over the block; the starts are then read from the
// LDS copy.  Otherwise two waves search off in global memory and the starts
// are copied into LDS.
__device__ void find_tile_layers(TileLayers& T, const int64_t (&o)[kOffPerThread],
                                 const int64_t* __restrict__ off, int nl,
                                 int64_t t0, int64_t t1, int& lf, int& ns) {
  __shared__ int ends[2];
  __shared__ int cnt[2][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (nl < kOffCache) {
    int c0 = 0, c1 = 0;
#pragma unroll
    for (int j = 0; j < kOffPerThread; ++j) {
      const int idx = threadIdx.x + 256 * j;
      if (idx <= nl) T.offc[idx] = o[j];
      if (idx >= 1 && idx < nl) {
        c0 += o[j] <= t0 ? 1 : 0;
        c1 += o[j] <= t1 - 1 ? 1 : 0;
      }
    }
    auto addi = [](int a, int b) { return a + b; };
    c0 = group_reduce<64>(c0, addi);
    c1 = group_reduce<64>(c1, addi);
    if (lane == 0) {
      cnt[0][wave] = c0;
      cnt[1][wave] = c1;
    }
    __syncthreads();
    lf = cnt[0][0] + cnt[0][1] + cnt[0][2] + cnt[0][3];
    const int ll = cnt[1][0] + cnt[1][1] + cnt[1][2] + cnt[1][3];
    ns = (ll < lf || ll - lf > kMaxStarts) ? -1 : ll - lf;
    return;
  }
  if (wave < 2) {
    const int l = layer_of_wave(off, nl, wave == 0 ? t0 : t1 - 1);
    if (lane == 0) ends[wave] = l;
  }
  __syncthreads();
  lf = ends[0];
  const int ll = ends[1];
  ns = (ll < lf || ll - lf > kMaxStarts) ? -1 : ll - lf;
  if (ns > 0 && (int)threadIdx.x < ns) T.starts[threadIdx.x] = off[lf + 1 + threadIdx.x];
  __syncthreads();
}

// Layer of flat element i of the tile (lf, ns from find_tile_layers).
__device__ __forceinline__ int elem_layer(const TileLayers& T, int lf, int ns,
                                          const int64_t* __restrict__ off,
                                          int nl, int64_t i) {
  if (ns == 0) return lf;
  if (ns < 0) return layer_of(nl < kOffCache ? T.offc : off, nl, i);
  const int64_t* st = nl < kOffCache ? T.offc + lf + 1 : T.starts;
  int lo = 0, hi = ns;  // count of starts <= i
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (st[mid] <= i) lo = mid + 1;
    else hi = mid;
  }
  return lf + lo;
}

}  // namespace gq

// ----------------------------------------------------- host launchers --
// Implemented in the kernel translation units; called by the C ABI after
// validation.  Each returns 0 or a hipError_t value.
namespace gq {

struct LaunchDesc {
  int scheme, d, s, L, flags, bits, k;
  float clip_sigma;
  // dense packing (when it differs from the fixed-width layout): alphabet
  // size A, A^4, and the field width W of 8 codes; dense = 0 otherwise
  int dense, A, W;
  uint32_t A4;
};

struct PayloadPtrs {
  const uint8_t* codes[kMaxPayloads];
  const float* meta[kMaxPayloads];
};

// quantize (codes != nullptr) or levels only (codes == nullptr, e read-only)
int launch_stream_quant(const LaunchDesc& L, int64_t n, const float* g,
                        float* e, uint64_t seed, uint32_t step, uint8_t* codes,
                        float* meta, int64_t code_bytes, hipStream_t st);
int launch_sort_quant(const LaunchDesc& L, int64_t n, const float* g, float* e,
                      uint64_t seed, uint32_t step, uint8_t* codes, float* meta,
                      int64_t code_bytes, hipStream_t st);
// BinGrad-b without sorting the bucket (bucket sizes 128 .. 2048); buckets it
// leaves unresolved get NaN levels and untouched codes and residuals.
bool binopt_prune_supported(int d);
int launch_binopt_prune(int d, int64_t n, const float* g, float* e,
                        uint8_t* codes, float* meta, int64_t code_bytes,
                        hipStream_t st);
int launch_deq_acc(const LaunchDesc& L, int64_t n, int W, const PayloadPtrs& pp,
                   float alpha, float beta, float* out, int64_t code_bytes,
                   hipStream_t st);
int launch_error_feedback(const LaunchDesc& L, int64_t n, const float* g,
                          float* e, const uint8_t* codes, const float* meta,
                          int64_t code_bytes, hipStream_t st);
// Top-K sparsification with quantization (d <= 512; L = K): record words per
// bucket, quantize (with the residual), dequantize-accumulate
int topk_record_words(int d, int bits, int K);
int launch_topk_quant(const LaunchDesc& L, int64_t n, const float* g, float* e,
                      uint64_t seed, uint32_t step, uint8_t* codes,
                      float* meta, hipStream_t st);
int launch_topk_deq(const LaunchDesc& L, int64_t n, int W, const PayloadPtrs& pp,
                    float alpha, float beta, float* out, hipStream_t st);
// Elias gamma coding of uniform-scheme codes: worst-case stream words,
// encode (three launches: counts, scan, records), decode (codes re-packed)
int64_t elias_max_words(const LaunchDesc& L, int64_t n);
int launch_elias_encode(const LaunchDesc& L, int64_t n, const uint8_t* codes,
                        uint64_t* off, uint32_t* words, hipStream_t st);
int launch_elias_decode(const LaunchDesc& L, int64_t n, const uint64_t* off,
                        const uint32_t* words, int64_t n_words, uint8_t* codes,
                        hipStream_t st);
// per-layer scale (uniform scheme): max-abs pass then rounding pass
// (codes == nullptr: the max-abs pass only)
int launch_layer_quant(const LaunchDesc& L, int64_t n, int nl,
                       const int64_t* off, const float* g, float* e,
                       uint64_t seed, uint32_t step, uint8_t* codes,
                       float* meta, int64_t code_bytes, hipStream_t st);
int launch_layer_alloc(int nl, const int64_t* off, const float* scales,
                       int64_t budget, int32_t* widths, int64_t* seg,
                       hipStream_t st);
// payload of a layer-wise bit allocation: max-abs pass, then the codes
// of each layer at its own width in its own segment (and the residual);
// dequantize-accumulate of W such payloads
int launch_alloc_quant(int64_t n, int nl, const int64_t* off, const float* g,
                       float* e, const int32_t* widths, const int64_t* seg,
                       uint64_t seed, uint32_t step, int nearest,
                       uint8_t* payload, int64_t payload_bytes, float* meta,
                       hipStream_t st);
int launch_alloc_deq(int64_t n, int nl, const int64_t* off, int W,
                     const uint8_t* const* pay, const float* const* meta,
                     const int32_t* const* widths, const int64_t* const* seg,
                     float alpha, float beta, float* out, hipStream_t st);
int launch_layer_deq(const LaunchDesc& L, int64_t n, int nl,
                     const int64_t* off, int W, const PayloadPtrs& pp,
                     float alpha, float beta, float* out, int64_t code_bytes,
                     hipStream_t st);

}  // namespace gq
