// layer_quant.hip — per-layer scale: TernGrad keeps one scaling factor per
// layer ("Gradient Quantization" glossary, ternary paragraph).  The flat
// gradient is the concatenation of nl layers, layer l = elements
// [off[l], off[l+1]), and each layer is one bucket of the uniform scheme of
// whatever size and offset.
//
// Two passes, because every code of a layer needs the layer's max-abs:
//   k_layer_absmax  p = g (+ e), max |p| per layer into meta (zeroed first
//                   by k_zero_u32; maxima of non-negative floats combine as
//                   unsigned integers), each block over a run of tiles;
//   k_layer_quant   p = g (+ e) again, random rounding with the element's
//                   layer scale, packing into the same flat stream as the
//                   bucketed layout, residual.
// Both walk the flat gradient in tiles of kLTile elements (thread t of a
// block owns float4 groups t and t + kLThreads, so each wave covers 256
// consecutive elements per pass, as the packing helpers require).  The
// layers that meet a tile are found once per block (find_tile_layers in
// common.hpp) and their constants kept in LDS.
#include "common.hpp"

namespace gq {
namespace {

constexpr int kLThreads = 256;
constexpr int kLV = 2;                            // float4 groups per thread
constexpr int kLGroups = kLThreads * kLV;         // groups per tile
constexpr int64_t kLTile = 4 * (int64_t)kLGroups;  // elements per tile
static_assert(kLThreads == 256, "find_tile_layers expects blocks of 256 threads");

__global__ void k_zero_u32(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// p = g (+ e) for the kLV groups of this thread in the tile starting at
// group tile_g (absent elements 0).  A tile wholly inside the gradient
// issues all its 128-bit nontemporal loads before any use; `between` runs
// while they are in flight.
template <typename F = void (*)()>
__device__ __forceinline__ void load_tile(float4 (&p)[kLV],
                                          const float* __restrict__ g,
                                          const float* __restrict__ e,
                                          int64_t tile_g, int64_t ngroups,
                                          int64_t n, F between = [] {}) {
  float4 r[kLV];
  if (4 * (tile_g + kLGroups) <= n) {
#pragma unroll
    for (int v = 0; v < kLV; ++v)
      p[v] = load4_nt(g + 4 * (tile_g + threadIdx.x + (int64_t)kLThreads * v));
    if (e != nullptr) {
#pragma unroll
      for (int v = 0; v < kLV; ++v)
        r[v] = load4_nt(e + 4 * (tile_g + threadIdx.x + (int64_t)kLThreads * v));
    }
    between();
  } else {
#pragma unroll
    for (int v = 0; v < kLV; ++v) {
      const int64_t f = tile_g + threadIdx.x + (int64_t)kLThreads * v;
      const bool live = f < ngroups;
      p[v] = live ? load4(g, 4 * f, n) : make_float4(0.f, 0.f, 0.f, 0.f);
      if (e != nullptr) r[v] = live ? load4(e, 4 * f, n) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    between();
  }
  if (e != nullptr) {
#pragma unroll
    for (int v = 0; v < kLV; ++v) {
      p[v].x = p[v].x + r[v].x;
      p[v].y = p[v].y + r[v].y;
      p[v].z = p[v].z + r[v].z;
      p[v].w = p[v].w + r[v].w;
    }
  }
}

// Blocks of the max-abs pass.  Each takes a contiguous run of tiles and
// keeps a running maximum for the layer it is in, updating meta only when
// the layer changes and at its end: one update per tile would queue up to
// thousands of atomics on the address of a large layer.
constexpr int64_t kAbsmaxBlocks = 4096;

__global__ __launch_bounds__(kLThreads) void k_layer_absmax(
    int64_t n, int nl, const int64_t* __restrict__ off,
    const float* __restrict__ g, const float* __restrict__ e,
    uint32_t* __restrict__ meta_bits) {
  __shared__ TileLayers T;
  __shared__ uint32_t smax[kMaxStarts + 1];
  const int64_t ngroups = (n + 3) >> 2;
  const int64_t ntiles = (n + kLTile - 1) / kLTile;
  const int64_t per = (ntiles + gridDim.x - 1) / gridDim.x;
  const int64_t tb = (int64_t)blockIdx.x * per;
  const int64_t te = tb + per < ntiles ? tb + per : ntiles;
  const int lane = threadIdx.x & 63;
  int64_t o[kOffPerThread];
  prefetch_offsets(o, off, nl);
  int cur_l = -1;       // thread 0: the running layer and its maximum
  uint32_t cur_m = 0u;

  for (int64_t tile = tb; tile < te; ++tile) {
    const int64_t tile_g = tile * kLGroups;
    const int64_t t0 = 4 * tile_g;
    const int64_t t1 = t0 + kLTile < n ? t0 + kLTile : n;
    // the data loads go out first; the layer search runs while they are in
    // flight
    float4 p[kLV];
    if ((int)threadIdx.x <= kMaxStarts) smax[threadIdx.x] = 0u;
    int lf = 0, ns = 0;
    load_tile(p, g, e, tile_g, ngroups, n,
              [&] { find_tile_layers(T, o, off, nl, t0, t1, lf, ns); });
#pragma unroll
    for (int v = 0; v < kLV; ++v) {
      const int64_t i = 4 * (tile_g + threadIdx.x + (int64_t)kLThreads * v);
      const float m = fmaxf(fmaxf(fabsf(p[v].x), fabsf(p[v].y)),
                            fmaxf(fabsf(p[v].z), fabsf(p[v].w)));
      if (ns == 0) {
        // the whole tile is one layer: one wave maximum, one LDS update
        const float wm = group_max<64>(m);
        if (lane == 0) atomicMax(&smax[0], __float_as_uint(wm));
      } else {
        // elements of several layers: each real element on its own (absent
        // ones load as 0 and never raise a maximum)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (i + k >= n) break;
          const uint32_t b = __float_as_uint(fabsf(comp(p[v], k)));
          if (b == 0u) continue;
          const int l = elem_layer(T, lf, ns, off, nl, i + k);
          if (ns > 0) atomicMax(&smax[l - lf], b);
          else atomicMax(&meta_bits[l], b);
        }
      }
    }
    __syncthreads();
    if (threadIdx.x == 0 && ns >= 0) {
      for (int k = 0; k <= ns; ++k) {
        const int l = lf + k;
        const uint32_t m = smax[k];
        if (l == cur_l) {
          cur_m = m > cur_m ? m : cur_m;
        } else {
          if (cur_l >= 0 && cur_m != 0u) atomicMax(&meta_bits[cur_l], cur_m);
          cur_l = l;
          cur_m = m;
        }
      }
    }
    __syncthreads();  // smax and T are rewritten by the next tile
  }
  if (threadIdx.x == 0 && cur_l >= 0 && cur_m != 0u) atomicMax(&meta_bits[cur_l], cur_m);
}

template <int BITS>
__global__ __launch_bounds__(kLThreads) void k_layer_quant(
    int64_t n, int nl, const int64_t* __restrict__ off,
    const float* __restrict__ g, float* __restrict__ e, uint32_t k0,
    uint32_t k1, uint32_t step, int s, int nearest, uint8_t* __restrict__ codes,
    const float* __restrict__ meta, int64_t code_bytes, uint32_t A4, int W) {
  constexpr bool DENSE = BITS == 0;
  __shared__ TileLayers T;
  __shared__ LayerScale sc[kMaxStarts + 1];
  const int64_t ngroups = (n + 3) >> 2;
  const int64_t tile_g = (int64_t)blockIdx.x * kLGroups;
  const int64_t t0 = 4 * tile_g;
  const int64_t t1 = t0 + kLTile < n ? t0 + kLTile : n;
  const float sf = (float)s;
  const int lane = threadIdx.x & 63;

  float4 p[kLV];
  uint4 wr[kLV];
  // random words (drawn while the loads are in flight), or (nearest) words
  // whose u is exactly 1/2
  auto draw = [&]() {
#pragma unroll
    for (int v = 0; v < kLV; ++v) {
      const uint64_t f = (uint64_t)(tile_g + threadIdx.x + (int64_t)kLThreads * v);
      wr[v] = nearest ? make_uint4(kHalfWord, kHalfWord, kHalfWord, kHalfWord)
                      : philox4x32_10(k0, k1, (uint32_t)f, (uint32_t)(f >> 32), step, 0u);
    }
  };
  // the random words and the layers of the tile are found while the data
  // loads are in flight (neither depends on them)
  int64_t o[kOffPerThread];
  prefetch_offsets(o, off, nl);
  int lf = 0, ns = 0;
  load_tile(p, g, e, tile_g, ngroups, n, [&] {
    draw();
    find_tile_layers(T, o, off, nl, t0, t1, lf, ns);
  });
  // a tile inside one layer (ns = 0, block-uniform) takes its layer's
  // constants without the LDS table and its barrier
  LayerScale c0{1.f, 0.f, 0.f};
  if (ns == 0) {
    c0 = layer_scale(meta[lf], sf);
  } else {
    if (ns > 0 && (int)threadIdx.x <= ns)
      sc[threadIdx.x] = layer_scale(meta[lf + threadIdx.x], sf);
    __syncthreads();
    if (ns > 0) c0 = sc[0];
  }

#pragma unroll
  for (int v = 0; v < kLV; ++v) {
    const int64_t f = tile_g + threadIdx.x + (int64_t)kLThreads * v;
    const int64_t i = 4 * f;
    const uint32_t ws[4] = {wr[v].x, wr[v].y, wr[v].z, wr[v].w};
    int sc4[4];
    float xh[4];
    const int nreal = i + 4 <= n ? 4 : (i < n ? (int)(n - i) : 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      LayerScale c = c0;
      if (ns != 0) {
        const int l = elem_layer(T, lf, ns, off, nl, i + k < n ? i + k : n - 1);
        c = ns > 0 ? sc[l - lf] : layer_scale(meta[l], sf);
      }
      const int ci = k < nreal ? uniform_code<true>(comp(p[v], k), c.up, c.inv, sf, ws[k]) : 0;
      sc4[k] = ci;
      xh[k] = (float)ci * c.delta;
    }
    if constexpr (DENSE) {
      const uint32_t A = 2u * (uint32_t)s + 1u;
      uint32_t u = 0u;
#pragma unroll
      for (int k = 3; k >= 0; --k)
        u = __umul24(u, A) + (k < nreal ? (uint32_t)(sc4[k] + s) : 0u);
      store_dense_chunk(codes, i - 4 * lane, u, A4, W, code_bytes);
    } else {
      constexpr uint32_t mask = (1u << BITS) - 1u;
      store_field<BITS, 64>(codes, i, lane,
                            field4<BITS>((uint32_t)sc4[0] & mask, (uint32_t)sc4[1] & mask,
                                         (uint32_t)sc4[2] & mask, (uint32_t)sc4[3] & mask),
                            code_bytes);
    }
    if (e != nullptr && i < n) {
      float4 r;
      r.x = p[v].x - xh[0];
      r.y = p[v].y - xh[1];
      r.z = p[v].z - xh[2];
      r.w = p[v].w - xh[3];
      if (nreal == 4) store4_nt(e + i, r);
      else store4(e, i, n, r);
    }
  }
}

// ------------------------------------------------ layer-wise bit allocation
// ("Gradient Quantization" glossary, layer-wise quantization paragraph:
// wider codes for layers with larger gradient variance).  One block: widths
// b in {2, 3, 4, 8} (s = 2^(b-1) - 1) start at 2; the 3 nl upgrades
// (2->3, 3->4, 4->8 of each layer) are sorted by the reduction of the
// layer's variance bound n_l M_l^2 / (4 s^2) per added bit,
// M_l^2 (1/s_b^2 - 1/s_b'^2) / (4 (b' - b)) in fp64, equal reductions by
// layer, then width (bitonic sort in LDS), and taken in that order up to the
// first that does not fit the budget of code bits; upgrades that reduce
// nothing end the list, those of empty layers are passed over.  Then each
// layer's code segment: its n_l codes at its width, padded to 16 bytes.
constexpr int kAllocThreads = 1024;
constexpr int kAllocMaxLayers = 1024;
constexpr int kAllocSlots = 4096;  // >= 3 * kAllocMaxLayers, a power of two

__device__ __forceinline__ double alloc_step_gain(float m, int k) {
  // k = 0, 1, 2: 2->3, 3->4, 4->8 (s = 1, 3, 7, 127)
  const double s0 = k == 0 ? 1.0 : (k == 1 ? 3.0 : 7.0);
  const double s1 = k == 0 ? 3.0 : (k == 1 ? 7.0 : 127.0);
  const double db = k == 2 ? 4.0 : 1.0;
  const double m2 = (double)m * (double)m;
  return m2 * ((1.0 / (s0 * s0) - 1.0 / (s1 * s1)) / (4.0 * db));
}

// Inclusive block scan of one int64 per thread (1024 threads): a shuffle
// scan in each wave, the 16 wave totals through LDS, one barrier.
__device__ int64_t alloc_block_scan(int64_t v, int64_t* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) tmp[wave] = v;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < wave; ++w) before += tmp[w];
  __syncthreads();  // tmp is reused by the next scan
  return v + before;
}

__global__ __launch_bounds__(kAllocThreads) void k_layer_alloc(
    int nl, const int64_t* __restrict__ off, const float* __restrict__ scales,
    int64_t budget, int32_t* __restrict__ widths, int64_t* __restrict__ seg) {
  __shared__ double gain[kAllocSlots];
  __shared__ int key[kAllocSlots];          // layer * 3 + step
  __shared__ int64_t scan[kAllocThreads / 64];
  __shared__ int wid[kAllocMaxLayers];
  __shared__ int64_t nsz[kAllocMaxLayers];
  __shared__ int first_stop;
  __shared__ int64_t used_sh;
  const int t = threadIdx.x;
  if (t < nl) {
    const int64_t a = off[t], b = off[t + 1];
    nsz[t] = b > a ? b - a : 0;
    wid[t] = 2;
  }
  if (t == 0) first_stop = kAllocSlots;
  for (int i = t; i < kAllocSlots; i += kAllocThreads) {
    const int lay = i / 3;
    if (lay < nl) {
      gain[i] = alloc_step_gain(scales[lay], i % 3);
      key[i] = i;
    } else {
      gain[i] = -1.0;  // padding sorts last (real gains are >= 0)
      key[i] = 0x7fffffff;
    }
  }
  __syncthreads();
  // bitonic sort of the first P slots (P: the power of two >= 3 nl; the
  // rest is padding already in place): larger gain first, then smaller key
  int P = 1;
  while (P < 3 * nl) P <<= 1;
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = t; i < P; i += kAllocThreads) {
        const int p = i ^ j;
        if (p > i) {
          const bool before_ip = gain[i] > gain[p] || (gain[i] == gain[p] && key[i] < key[p]);
          const bool want = (i & k) == 0;  // this run ascending in "before"
          if (before_ip != want) {
            const double g0 = gain[i];
            gain[i] = gain[p];
            gain[p] = g0;
            const int k0 = key[i];
            key[i] = key[p];
            key[p] = k0;
          }
        }
      }
      __syncthreads();
    }
  }
  // costs in sorted order (4 slots per thread), their running total, and
  // the first slot that ends the list (no reduction, or over the budget)
  // bits of every layer at 2: the block's total, from the last thread
  {
    const int64_t incl = alloc_block_scan(t < nl ? 2 * nsz[t] : 0, scan);
    if (t == kAllocThreads - 1) used_sh = incl;
    __syncthreads();
  }
  const int64_t used0 = used_sh;
  int64_t c[4];
  int64_t loc = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 4 * t + q;
    const int kk = key[i];
    int64_t cost = 0;
    if (kk != 0x7fffffff) {
      const int lay = kk / 3, st = kk % 3;
      cost = nsz[lay] * (st == 2 ? 4 : 1);
    }
    loc += cost;
    c[q] = loc;
  }
  const int64_t excl = alloc_block_scan(loc, scan) - loc;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 4 * t + q;
    const bool stop = !(gain[i] > 0.0) || used0 + excl + c[q] > budget;
    if (stop) atomicMin(&first_stop, i);
  }
  __syncthreads();
  const int fs = first_stop;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 4 * t + q;
    if (i < fs) {
      const int kk = key[i];
      const int lay = kk / 3, st = kk % 3;
      if (nsz[lay] > 0) atomicMax(&wid[lay], st == 0 ? 3 : (st == 1 ? 4 : 8));
    }
  }
  __syncthreads();
  // segments: each layer's codes at its width, padded to 16 bytes
  int64_t bytes = 0;
  if (t < nl) {
    widths[t] = wid[t];
    bytes = ((nsz[t] * wid[t] + 7) / 8 + 15) / 16 * 16;
  }
  const int64_t incl = alloc_block_scan(bytes, scan);
  if (t < nl) seg[t + 1] = incl;
  if (t == 0) seg[0] = 0;
}

}  // namespace

int launch_layer_alloc(int nl, const int64_t* off, const float* scales,
                       int64_t budget, int32_t* widths, int64_t* seg,
                       hipStream_t st) {
  if (nl < 1 || nl > kAllocMaxLayers) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_layer_alloc, dim3(1), dim3(kAllocThreads), 0, st, nl,
                     off, scales, budget, widths, seg);
  return (int)hipGetLastError();
}

int launch_layer_quant(const LaunchDesc& L, int64_t n, int nl,
                       const int64_t* off, const float* g, float* e,
                       uint64_t seed, uint32_t step, uint8_t* codes,
                       float* meta, int64_t code_bytes, hipStream_t st) {
  const int64_t tiles = (n + kLTile - 1) / kLTile;
  hipLaunchKernelGGL(k_zero_u32, dim3((uint32_t)((nl + 255) / 256)), dim3(256),
                     0, st, reinterpret_cast<uint32_t*>(meta), (int64_t)nl);
  hipLaunchKernelGGL(k_layer_absmax,
                     dim3((uint32_t)(tiles < kAbsmaxBlocks ? tiles : kAbsmaxBlocks)),
                     dim3(kLThreads), 0, st, n, nl, off, g, e,
                     reinterpret_cast<uint32_t*>(meta));
  if (codes == nullptr) return (int)hipGetLastError();
  const int nearest = (L.flags & GQ_FLAG_NEAREST) ? 1 : 0;
#define GQ_LQ(BITS)                                                           \
  hipLaunchKernelGGL((k_layer_quant<BITS>), dim3((uint32_t)tiles),            \
                     dim3(kLThreads), 0, st, n, nl, off, g, e, (uint32_t)seed, \
                     (uint32_t)(seed >> 32), step, L.s, nearest, codes, meta, \
                     code_bytes, L.A4, L.W)
  if (L.dense) GQ_LQ(0);
  else if (L.bits == 2) GQ_LQ(2);
  else if (L.bits == 3) GQ_LQ(3);
  else if (L.bits == 4) GQ_LQ(4);
  else if (L.bits == 8) GQ_LQ(8);
  else return (int)hipErrorInvalidValue;
#undef GQ_LQ
  return (int)hipGetLastError();
}

}  // namespace gq
