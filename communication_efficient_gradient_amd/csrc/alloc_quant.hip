// alloc_quant.hip — the payload of a layer-wise bit allocation ("Gradient
// Quantization" glossary, layer-wise quantization paragraph: layers whose
// gradients vary more get wider codes).  Layer l holds elements
// [off[l], off[l+1]) and is coded at widths[l] bits, b in {2, 3, 4, 8}, with
// the uniform max-abs scheme at s = 2^(b-1) - 1 and one scale per layer
// (its max-abs, computed by the per-layer max-abs pass).  Its n_l codes
// form an LSB-first bit stream (code k at bits [k b, k b + b)) that starts
// at byte seg[l] of the payload; seg[] pads every segment to 16 bytes.
//
// The random word of element i is the one the other paths use (Philox
// counter i / 4, word i mod 4), so a layer's codes are exactly those of the
// per-layer path at that layer's s.
//
//   k_alloc_quant  one thread per 32-bit payload word, its codes and their
//                  residuals (at 3 bits, where codes straddle words, the
//                  thread of every third word takes three words: 32 whole
//                  codes, so no code is shared).  The grid covers the
//                  caller's payload capacity, so every store is in bounds
//                  whatever the segment table holds; threads past seg[nl]
//                  return.
//   k_alloc_deq    one thread per float4 of the output: for each payload the
//                  element's layer width, segment and step, the field read
//                  from one aligned word (two when it straddles), summed over
//                  the payloads as the per-layer dequantizer does.
#include "common.hpp"

namespace gq {
namespace {

constexpr int kAThreads = 256;

__device__ __forceinline__ bool alloc_width_ok(int b) {
  return b == 2 || b == 3 || b == 4 || b == 8;
}

// index l of the layer holding position x: off[l] <= x < off[l+1]
// (0 <= x < off[nl]; empty layers are never returned)
__device__ __forceinline__ int layer_of(const int64_t* __restrict__ off, int nl,
                                        int64_t x) {
  int lo = 0, hi = nl;  // off[lo] <= x < off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= x) lo = mid;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kAThreads) void k_alloc_quant(
    int64_t n, int nl, const int64_t* __restrict__ off, const float* __restrict__ g,
    float* __restrict__ e, const int32_t* __restrict__ widths,
    const int64_t* __restrict__ seg, uint32_t k0, uint32_t k1, uint32_t step,
    int nearest, uint32_t* __restrict__ payload, int64_t cap_words,
    const float* __restrict__ meta) {
  const int64_t w = (int64_t)blockIdx.x * kAThreads + threadIdx.x;
  if (w >= cap_words) return;
  const int64_t total = seg[nl];
  if (4 * w >= total) return;
  const int l = layer_of(seg, nl, 4 * w);
  const int b = widths[l];
  if (!alloc_width_ok(b)) {
    payload[w] = 0u;
    return;
  }
  // 3-bit codes straddle words: one thread takes three words (32 codes),
  // so every code, and its residual, belongs to one thread
  const int nw = b == 3 ? 3 : 1;
  const int64_t sw0 = seg[l] >> 2, sw1 = seg[l + 1] >> 2;
  if ((w - sw0) % nw != 0) return;
  const int64_t lo = off[l];
  const int64_t nlay = off[l + 1] - lo;
  const int64_t kfirst = 32 * (w - sw0) / b;  // first code of the group
  int64_t kend = kfirst + 32 * nw / b;
  if (kend > nlay) kend = nlay;
  if (lo < 0) kend = kfirst;           // offsets outside [0, n] read nothing
  else if (kend > n - lo) kend = n - lo;
  const int s = (1 << (b - 1)) - 1;
  const float sf = (float)s;
  const uint32_t mask = (1u << b) - 1u;
  const LayerScale c = layer_scale(meta[l], sf);
  uint64_t acc0 = 0u, acc1 = 0u;  // bits 0..63 and 64..127 of the group
  int64_t cur = -1;
  uint4 r = make_uint4(0u, 0u, 0u, 0u);
  for (int64_t k = kfirst; k < kend; ++k) {
    const int64_t i = lo + k;
    const int64_t f = i >> 2;
    if (!nearest && f != cur) {
      r = philox4x32_10(k0, k1, (uint32_t)f, (uint32_t)(f >> 32), step, 0u);
      cur = f;
    }
    const int q = (int)(i & 3);
    const uint32_t u = nearest ? kHalfWord : (q == 0 ? r.x : q == 1 ? r.y : q == 2 ? r.z : r.w);
    const float gi = g[i];
    const float p = e != nullptr ? gi + e[i] : gi;
    const int ci = uniform_code<true>(p, c.up, c.inv, sf, u);
    const uint64_t fld = (uint64_t)((uint32_t)ci & mask);
    const int pos = (int)((k - kfirst) * b);  // 0 .. 32 nw - b
    if (pos < 64) {
      acc0 |= fld << pos;
      if (pos + b > 64) acc1 |= fld >> (64 - pos);
    } else {
      acc1 |= fld << (pos - 64);
    }
    if (e != nullptr) e[i] = p - (float)ci * c.delta;
  }
  payload[w] = (uint32_t)acc0;
  if (nw == 3) {
    // the group may run past the segment's padded end (or the capacity)
    if (w + 1 < sw1 && w + 1 < cap_words) payload[w + 1] = (uint32_t)(acc0 >> 32);
    if (w + 2 < sw1 && w + 2 < cap_words) payload[w + 2] = (uint32_t)acc1;
  }
}

struct AllocPtrs {
  const uint32_t* pay[kMaxPayloads];
  const float* meta[kMaxPayloads];
  const int32_t* widths[kMaxPayloads];
  const int64_t* seg[kMaxPayloads];
};

__device__ __forceinline__ float alloc_value(const AllocPtrs& P, int p, int l,
                                             int64_t k) {
  const int b = P.widths[p][l];
  if (!alloc_width_ok(b)) return 0.f;
  const int s = (1 << (b - 1)) - 1;
  const int64_t bit = 8 * P.seg[p][l] + k * b;
  const uint32_t* wp = P.pay[p] + (bit >> 5);
  const int sh = (int)(bit & 31);
  uint32_t v = wp[0] >> sh;
  if (sh + b > 32) v |= wp[1] << (32 - sh);
  const int code = (int)(v << (32 - b)) >> (32 - b);  // sign-extend b bits
  return (float)code * (P.meta[p][l] / (float)s);
}

__global__ __launch_bounds__(kAThreads) void k_alloc_deq(
    int64_t n, int nl, const int64_t* __restrict__ off, int W, AllocPtrs P,
    float alpha, float beta, float* __restrict__ out) {
  const int64_t f = (int64_t)blockIdx.x * kAThreads + threadIdx.x;
  const int64_t i0 = 4 * f;
  if (i0 >= n) return;
  const int nreal = i0 + 4 <= n ? 4 : (int)(n - i0);
  int li[4];
  int l = layer_of(off, nl, i0);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k < nreal)
      while (l + 1 < nl && off[l + 1] <= i0 + k) ++l;
    li[k] = l;
  }
  float a0[4] = {0.f, 0.f, 0.f, 0.f}, a1[4] = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < W; ++p) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k >= nreal) continue;
      const float x = alloc_value(P, p, li[k], i0 + k - off[li[k]]);
      if (p == 0) a0[k] = x;
      else if (p == 1) a1[k] = x;
      else if (p & 1) a1[k] = a1[k] + x;
      else a0[k] = a0[k] + x;
    }
  }
  float r[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = W > 1 ? a0[k] + a1[k] : a0[k];
    r[k] = alpha * a;
  }
  if (nreal == 4) {
    float4 rv = make_float4(r[0], r[1], r[2], r[3]);
    if (beta != 0.f) {
      const float4 old = *reinterpret_cast<const float4*>(out + i0);
      rv.x = rv.x + beta * old.x;
      rv.y = rv.y + beta * old.y;
      rv.z = rv.z + beta * old.z;
      rv.w = rv.w + beta * old.w;
    }
    *reinterpret_cast<float4*>(out + i0) = rv;
  } else {
    for (int k = 0; k < nreal; ++k) {
      float rk = r[k];
      if (beta != 0.f) rk = rk + beta * out[i0 + k];
      out[i0 + k] = rk;
    }
  }
}

}  // namespace

int launch_alloc_quant(int64_t n, int nl, const int64_t* off, const float* g,
                       float* e, const int32_t* widths, const int64_t* seg,
                       uint64_t seed, uint32_t step, int nearest,
                       uint8_t* payload, int64_t payload_bytes, float* meta,
                       hipStream_t st) {
  // the layers' max-abs (the per-layer path's first pass)
  LaunchDesc L{};
  int rc = launch_layer_quant(L, n, nl, off, g, e, seed, step, nullptr, meta, 0, st);
  if (rc) return rc;
  const int64_t cap_words = payload_bytes / 4;
  const int64_t blocks = (cap_words + kAThreads - 1) / kAThreads;
  hipLaunchKernelGGL(k_alloc_quant, dim3((uint32_t)blocks), dim3(kAThreads), 0,
                     st, n, nl, off, g, e, widths, seg, (uint32_t)seed,
                     (uint32_t)(seed >> 32), step, nearest,
                     reinterpret_cast<uint32_t*>(payload), cap_words, meta);
  return (int)hipGetLastError();
}

int launch_alloc_deq(int64_t n, int nl, const int64_t* off, int W,
                     const uint8_t* const* pay, const float* const* meta,
                     const int32_t* const* widths, const int64_t* const* seg,
                     float alpha, float beta, float* out, hipStream_t st) {
  if (W < 1 || W > kMaxPayloads) return (int)hipErrorInvalidValue;
  AllocPtrs P{};
  for (int p = 0; p < W; ++p) {
    P.pay[p] = reinterpret_cast<const uint32_t*>(pay[p]);
    P.meta[p] = meta[p];
    P.widths[p] = widths[p];
    P.seg[p] = seg[p];
  }
  const int64_t groups = (n + 3) / 4;
  const int64_t blocks = (groups + kAThreads - 1) / kAThreads;
  hipLaunchKernelGGL(k_alloc_deq, dim3((uint32_t)blocks), dim3(kAThreads), 0,
                     st, n, nl, off, W, P, alpha, beta, out);
  return (int)hipGetLastError();
}

}  // namespace gq
