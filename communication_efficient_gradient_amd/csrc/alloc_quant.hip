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
                                        int64_t x, int lo = 0) {
  int hi = nl;  // off[lo] <= x < off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= x) lo = mid;
    else hi = mid;
  }
  return lo;
}

// The same search by a whole wave (every lane passes the same x): each
// round one load per lane at 64 evenly spaced candidates, so 160 layers take
// two rounds of one memory latency each instead of eight.
__device__ __forceinline__ int wave_layer_of(const int64_t* __restrict__ off,
                                             int nl, int64_t x) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = nl;  // off[lo] <= x < off[hi]
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const bool le = idx < hi && off[idx] <= x;  // true for a prefix of lanes
    const int cnt = __popcll(__ballot(le));     // >= 1: lane 0 reads off[lo]
    lo += (cnt - 1) * step;
    hi = lo + step < hi ? lo + step : hi;
  }
  return lo;
}

// LDS slot of staged element s: one pad word every 16 keeps the lanes of a
// strided read (16 consecutive elements per lane at 2 bits) on distinct banks
__device__ __forceinline__ int stage_slot(int s) { return s + (s >> 4); }

constexpr int kWaveElems = 1024;  // elements one wave codes at most (2 bits)

// The codes of one lane at width B: CNT = 32 nw / B consecutive codes of
// its layer, elements [i0, i0 + nreal) of the flat gradient, whose p the
// wave has staged in LDS (sp = that row, from element e_lo; -1 entries:
// outside the staged run, code 0).  Residuals go back to the same slots.
template <int B, int A>
__device__ __forceinline__ void alloc_quant_group(
    float* sp, int64_t e_lo, int64_t i0, int nreal, uint32_t k0, uint32_t k1,
    uint32_t step, int nearest, const LayerScale& c,
    uint32_t* __restrict__ payload, int64_t w, int64_t sw1, int64_t cap_words,
    bool ef) {
  constexpr int NW = B == 3 ? 3 : 1;
  constexpr int CNT = 32 * NW / B;
  constexpr int NF = CNT / 4 + 1;  // Philox counters the run can touch
  constexpr int S = (1 << (B - 1)) - 1;
  constexpr uint32_t MASK = (1u << B) - 1u;
  const float sf = (float)S;
  const int64_t r0 = i0 - e_lo;  // first slot in the staged row
  const int64_t f0 = i0 >> 2;
  uint32_t rw[4 * NF];
#pragma unroll
  for (int q = 0; q < NF; ++q) {
    const int64_t f = f0 + q;
    const uint4 r = nearest ? make_uint4(kHalfWord, kHalfWord, kHalfWord, kHalfWord)
                            : philox4x32_10(k0, k1, (uint32_t)f, (uint32_t)(f >> 32), step, 0u);
    rw[4 * q] = r.x;
    rw[4 * q + 1] = r.y;
    rw[4 * q + 2] = r.z;
    rw[4 * q + 3] = r.w;
  }
  // A = i0 mod 4, the word of element i0 within its counter (a template
  // argument, so that rw is indexed statically and stays in registers)
  uint32_t wd[NW];
#pragma unroll
  for (int m = 0; m < NW; ++m) wd[m] = 0u;
#pragma unroll
  for (int j = 0; j < CNT; ++j) {
    const int64_t slot = r0 + j;
    const bool live = j < nreal && slot >= 0 && slot < kWaveElems;
    const float p = live ? sp[stage_slot((int)slot)] : 0.f;
    const uint32_t u = rw[A + j];
    const int ci = live ? uniform_code<true>(p, c.up, c.inv, sf, u) : 0;
    const uint32_t fld = (uint32_t)ci & MASK;
    const int pos = j * B;
    wd[pos >> 5] |= fld << (pos & 31);
    if ((pos & 31) + B > 32) wd[(pos >> 5) + 1] |= fld >> (32 - (pos & 31));
    if (ef && live) sp[stage_slot((int)slot)] = p - (float)ci * c.delta;
  }
  payload[w] = wd[0];
#pragma unroll
  for (int m = 1; m < NW; ++m)  // the group may run past the segment's end
    if (w + m < sw1 && w + m < cap_words) payload[w + m] = wd[m];
}

__global__ __launch_bounds__(kAThreads) void k_alloc_quant(
    int64_t n, int nl, const int64_t* __restrict__ off, const float* __restrict__ g,
    float* __restrict__ e, const int32_t* __restrict__ widths,
    const int64_t* __restrict__ seg, uint32_t k0, uint32_t k1, uint32_t step,
    int nearest, uint32_t* __restrict__ payload, int64_t cap_words,
    const float* __restrict__ meta) {
  __shared__ float stage[kAThreads / 64][kWaveElems + kWaveElems / 16];
  const int lane = threadIdx.x & 63;
  float* sp = stage[threadIdx.x >> 6];
  const int64_t w = (int64_t)blockIdx.x * kAThreads + threadIdx.x;
  const int64_t total = seg[nl];
  // blocks wholly past the payload (the grid covers the capacity) leave at
  // once, before any barrier (block-uniform)
  if (4 * ((int64_t)blockIdx.x * kAThreads) >= total) return;
  // this lane's layer, width and run of elements (empty for lanes past the
  // payload, the second and third words of a 3-bit group, padding words)
  const bool word = w < cap_words && 4 * w < total;
  // the layer of the wave's first word, searched by the whole wave; a lane
  // past that layer searches on from there
  const int64_t wfirst = w - (threadIdx.x & 63);
  const int lw = 4 * wfirst < total ? wave_layer_of(seg, nl, 4 * wfirst) : 0;
  int l = 0, b = 0;
  int64_t sw1 = 0, i0 = 0, i1 = 0;
  float mx = 0.f;
  bool lead = false;
  if (word) {
    // the tables of the wave's layer loaded together (one memory latency),
    // again for the layer of a lane past it
    l = lw;
    int64_t s0 = seg[l], s1 = seg[l + 1], o0 = off[l], o1 = off[l + 1];
    b = widths[l];
    mx = meta[l];
    if (s1 <= 4 * w) {
      l = layer_of(seg, nl, 4 * w, l + 1);
      s0 = seg[l];
      s1 = seg[l + 1];
      o0 = off[l];
      o1 = off[l + 1];
      b = widths[l];
      mx = meta[l];
    }
    const int64_t sw0 = s0 >> 2;
    sw1 = s1 >> 2;
    if (!alloc_width_ok(b)) {
      payload[w] = 0u;
    } else {
      // 3-bit codes straddle words: one lane takes three words (32 codes),
      // so every code, and its residual, belongs to one lane
      const int nw = b == 3 ? 3 : 1;
      lead = (w - sw0) % nw == 0;
      if (lead) {
        const int64_t lo = o0;
        const int64_t nlay = o1 - lo;
        const int64_t kfirst = 32 * (w - sw0) / b;
        int64_t kend = kfirst + 32 * nw / b;
        if (kend > nlay) kend = nlay;
        if (lo < 0) kend = kfirst;  // offsets outside [0, n] read nothing
        else if (kend > n - lo) kend = n - lo;
        if (kend < kfirst) kend = kfirst;
        i0 = lo + kfirst;
        i1 = lo + kend;
      }
    }
  }
  // the wave's runs are consecutive (layers follow each other in both the
  // gradient and the payload): stage [first run's start, last run's end)
  const uint64_t busy = __ballot(lead && i1 > i0);
  int64_t e_lo = 0, e_hi = 0;
  if (busy != 0) {
    const int first = __ffsll((long long)busy) - 1;
    const int last = 63 - __clzll((long long)busy);
    e_lo = __shfl(i0, first, 64);
    e_hi = __shfl(i1, last, 64);
    if (e_hi > e_lo + kWaveElems) e_hi = e_lo + kWaveElems;
  }
  if (busy != 0) {
    // in chunks of eight rows of 64 (wave-uniform; chunks past the run are
    // skipped): a chunk's sixteen loads are issued before any is used, the
    // indexes past the run clamped to its last element (in bounds, the same
    // cache line) and only the LDS writes predicated.  Holding all sixteen
    // rows at once took 112 VGPRs (4 waves per SIMD).
    const int nrows = (int)((e_hi - e_lo + 63) >> 6);
#pragma unroll
    for (int c = 0; c < kWaveElems / 64; c += 8) {
      if (c < nrows) {
        float gv[8], ev[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int64_t i = e_lo + 64 * (c + t) + lane;
          gv[t] = g[i < e_hi ? i : e_hi - 1];
        }
        if (e != nullptr) {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int64_t i = e_lo + 64 * (c + t) + lane;
            ev[t] = e[i < e_hi ? i : e_hi - 1];
          }
#pragma unroll
          for (int t = 0; t < 8; ++t) gv[t] = gv[t] + ev[t];
        }
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (e_lo + 64 * (c + t) + lane < e_hi) sp[stage_slot(64 * (c + t) + lane)] = gv[t];
      }
    }
  }
  __syncthreads();
  if (lead) {
    const int nreal = (int)(i1 - i0);
    const LayerScale c = layer_scale(mx, (float)((1 << (b - 1)) - 1));
    const bool ef = e != nullptr;
#define GQ_AQ(B, A)                                                          \
  alloc_quant_group<B, A>(sp, e_lo, i0, nreal, k0, k1, step, nearest, c,     \
                          payload, w, sw1, cap_words, ef)
#define GQ_AQ4(B)                     \
  switch ((int)(i0 & 3)) {            \
    case 0: GQ_AQ(B, 0); break;       \
    case 1: GQ_AQ(B, 1); break;       \
    case 2: GQ_AQ(B, 2); break;       \
    default: GQ_AQ(B, 3); break;      \
  }
    switch (b) {
      case 2: GQ_AQ4(2); break;
      case 3: GQ_AQ4(3); break;
      case 4: GQ_AQ4(4); break;
      default: GQ_AQ4(8); break;
    }
#undef GQ_AQ4
#undef GQ_AQ
  }
  __syncthreads();
  if (e != nullptr) {
#pragma unroll
    for (int t = 0; t < kWaveElems / 64; ++t) {
      const int64_t i = e_lo + 64 * t + lane;
      if (i < e_hi) e[i] = sp[stage_slot(64 * t + lane)];
    }
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

constexpr int kDeqV = 4;  // float4 groups per thread

// One float4 group of the output, elements [i0, i0 + 4) (those at or past n
// absent); l: a layer at or before that of i0 (off[l] <= i0).
__device__ __forceinline__ void alloc_deq_group(
    int64_t n, int nl, const int64_t* __restrict__ off, int W, const AllocPtrs& P,
    float alpha, float beta, float* __restrict__ out, int64_t i0, int l) {
  const int nreal = i0 + 4 <= n ? 4 : (int)(n - i0);
  int li[4];
  if (off[l + 1] <= i0) l = layer_of(off, nl, i0, l + 1);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k < nreal)
      while (l + 1 < nl && off[l + 1] <= i0 + k) ++l;
    li[k] = l;
  }
  float a0[4] = {0.f, 0.f, 0.f, 0.f}, a1[4] = {0.f, 0.f, 0.f, 0.f};
  const bool one = li[0] == li[nreal - 1];
  const int64_t kl = i0 - off[li[0]];  // layer-relative index of element i0
  for (int p = 0; p < W; ++p) {
    float x[4];
    if (one) {
      // the four codes lie in one layer: one table lookup and a 64-bit
      // window of at most two payload words
      const int lq = li[0];
      const int b = P.widths[p][lq];
      const bool ok = alloc_width_ok(b);
      const int bb = ok ? b : 2;
      const int64_t bit = 8 * P.seg[p][lq] + kl * bb;
      const uint32_t* wp = P.pay[p] + (bit >> 5);
      const int sh = (int)(bit & 31);
      uint64_t v = ok ? wp[0] : 0u;
      if (ok && sh + nreal * bb > 32) v |= (uint64_t)wp[1] << 32;
      const float delta = P.meta[p][lq] / (float)((1 << (bb - 1)) - 1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t fld = (uint32_t)(v >> (sh + k * bb));
        const int code = (int)(fld << (32 - bb)) >> (32 - bb);
        x[k] = ok ? (float)code * delta : 0.f;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        x[k] = k < nreal ? alloc_value(P, p, li[k], i0 + k - off[li[k]]) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (p == 0) a0[k] = x[k];
      else if (p == 1) a1[k] = x[k];
      else if (p & 1) a1[k] = a1[k] + x[k];
      else a0[k] = a0[k] + x[k];
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

__global__ __launch_bounds__(kAThreads) void k_alloc_deq(
    int64_t n, int nl, const int64_t* __restrict__ off, int W, AllocPtrs P,
    float alpha, float beta, float* __restrict__ out) {
  // thread t of a block owns groups t, t + 256, t + 512, t + 768 of the
  // block's 1024; the layer of the wave's first element is searched by the
  // whole wave and each group's search starts there (and is skipped when
  // its four elements lie in that layer)
  const int64_t f0 = (int64_t)blockIdx.x * kAThreads * kDeqV + threadIdx.x;
  const int l0 = wave_layer_of(off, nl, 4 * (f0 - (threadIdx.x & 63)));
  const int64_t ilast = 4 * (f0 + (int64_t)kAThreads * (kDeqV - 1)) + 3;
  // the first payload's tables for that layer are loaded with the layer's
  // end (they depend on l0 alone), one memory latency for both
  const int64_t end0 = off[l0 + 1];
  const int b0 = P.widths[0][l0];
  const int64_t seg0 = P.seg[0][l0];
  const float m0 = P.meta[0][l0];
  if (ilast < n && ilast < end0) {
    // all sixteen elements in layer l0: per payload one table lookup, and
    // the four groups' payload windows loaded together
    const int64_t base = 4 * f0 - off[l0];  // layer-relative index, group 0
    float a0[kDeqV][4], a1[kDeqV][4];
    for (int p = 0; p < W; ++p) {
      const int b = p == 0 ? b0 : P.widths[p][l0];
      const bool ok = alloc_width_ok(b);
      const int bb = ok ? b : 2;
      const int64_t bit0 = 8 * (p == 0 ? seg0 : P.seg[p][l0]);
      const float delta = (p == 0 ? m0 : P.meta[p][l0]) / (float)((1 << (bb - 1)) - 1);
      uint64_t win[kDeqV];
      int sh[kDeqV];
#pragma unroll
      for (int v = 0; v < kDeqV; ++v) {
        const int64_t bit = bit0 + (base + 4 * kAThreads * v) * bb;
        const uint32_t* wp = P.pay[p] + (bit >> 5);
        sh[v] = (int)(bit & 31);
        win[v] = ok ? wp[0] : 0u;
        if (ok && sh[v] + 4 * bb > 32) win[v] |= (uint64_t)wp[1] << 32;
      }
#pragma unroll
      for (int v = 0; v < kDeqV; ++v) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t fld = (uint32_t)(win[v] >> (sh[v] + k * bb));
          const int code = (int)(fld << (32 - bb)) >> (32 - bb);
          const float x = ok ? (float)code * delta : 0.f;
          if (p == 0) a0[v][k] = x;
          else if (p == 1) a1[v][k] = x;
          else if (p & 1) a1[v][k] = a1[v][k] + x;
          else a0[v][k] = a0[v][k] + x;
        }
      }
    }
#pragma unroll
    for (int v = 0; v < kDeqV; ++v) {
      const int64_t i0 = 4 * (f0 + (int64_t)kAThreads * v);
      float r[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) r[k] = alpha * (W > 1 ? a0[v][k] + a1[v][k] : a0[v][k]);
      float4 rv = make_float4(r[0], r[1], r[2], r[3]);
      if (beta != 0.f) {
        const float4 old = *reinterpret_cast<const float4*>(out + i0);
        rv.x = rv.x + beta * old.x;
        rv.y = rv.y + beta * old.y;
        rv.z = rv.z + beta * old.z;
        rv.w = rv.w + beta * old.w;
      }
      *reinterpret_cast<float4*>(out + i0) = rv;
    }
    return;
  }
#pragma unroll
  for (int v = 0; v < kDeqV; ++v) {
    const int64_t i0 = 4 * (f0 + (int64_t)kAThreads * v);
    if (i0 < n) alloc_deq_group(n, nl, off, W, P, alpha, beta, out, i0, l0);
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
  const int64_t blocks = (groups + kAThreads * kDeqV - 1) / (kAThreads * kDeqV);
  hipLaunchKernelGGL(k_alloc_deq, dim3((uint32_t)blocks), dim3(kAThreads), 0,
                     st, n, nl, off, W, P, alpha, beta, out);
  return (int)hipGetLastError();
}

}  // namespace gq
