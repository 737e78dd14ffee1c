// elias.hip — Elias gamma coding of uniform-scheme codes, the lossless step
// QSGD applies to its quantized integers ("Gradient Quantization" glossary,
// QSGD paragraph).  Code c becomes gamma(m), m = |c| + 1 (floor(log2 m)
// zeros, then the digits of m from the most significant), then a sign bit
// (1 = negative) when c != 0.  Each bucket's record starts on a 32-bit word;
// off[j] is the first word of record j and off[nb] the stream's length.
//
// Encode: three launches, no scratch memory.
//   1. k_elias_count: a block owns kChunk consecutive buckets, a wave one
//      bucket at a time.  Each bucket's word count, then the chunk's
//      inclusive scan: off[j + 1] = words of the chunk's buckets up to j.
//   2. k_elias_scan: one block turns the chunk totals (each sits at its
//      chunk's last entry) into global inclusive sums in place; off[0] = 0.
//   3. k_elias_write: one wave per bucket.  Its record starts at
//      off[chunk start] + off[j] (entries at chunk starts are final after
//      step 2; the wave writes the final off[j] back).  Per segment of 64 G
//      elements, lane l takes G consecutive codes, a wave scan of their bit
//      counts places them, each lane ORs its bits into the wave's LDS window
//      32 at a time, and the segment's whole words go out; the last partial
//      word carries into the next segment.
// Decode: one lane per bucket parses its record serially from a 64-bit
// window kept above 32 bits from a ring of kLook words loaded ahead, and
// packs the codes back into the fixed-width layout 32 bits at a time.
#include "common.hpp"

namespace gq {
namespace {

constexpr int kWaves = 4;     // waves per block (count and write passes)
constexpr int kChunk = 64;    // buckets per block in the count pass
constexpr int kScan = 1024;   // threads of the one-block scan
constexpr int kLook = 4;      // decode: words loaded ahead of the window

__device__ __forceinline__ int sext_clamp(uint32_t raw, int b, int s) {
  const int c = (int)(raw << (32 - b)) >> (32 - b);
  return c < -s ? -s : (c > s ? s : c);
}

// The gamma codeword of |c| + 1 and the sign, as stream bits from bit 0.
__device__ __forceinline__ uint32_t gamma_field(int c, int& len) {
  const uint32_t m = (uint32_t)(c < 0 ? -c : c) + 1u;
  const int L = 31 - __clz((int)m);
  len = c == 0 ? 1 : 2 * L + 2;
  return ((__brev(m) >> (31 - L)) << L) | ((c < 0 ? 1u : 0u) << (2 * L + 1));
}

// Bits [pos, pos + nbits) of the fixed-width code stream, nbits <= 64 - pos % 32.
__device__ __forceinline__ uint64_t stream_bits(const uint32_t* __restrict__ w,
                                                int64_t pos, int nbits) {
  const int64_t q = pos >> 5;
  const int sh = (int)(pos & 31);
  uint64_t v = w[q];
  if (sh + nbits > 32) v |= (uint64_t)w[q + 1] << 32;
  return v >> sh;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = (uint32_t)__shfl_up((int)v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Lane's G codes of a segment: count of live ones and their gamma fields.
template <int G>
__device__ __forceinline__ int lane_fields(const uint32_t* __restrict__ codes,
                                           int64_t e0, int ge, int b, int s,
                                           uint32_t (&f)[G], int (&l)[G]) {
  uint64_t x = 0;
  if (ge > 0) x = stream_bits(codes, e0 * b, ge * b);
  const uint32_t mask = (1u << b) - 1u;
  int tot = 0;
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const int c = sext_clamp((uint32_t)(x >> (k * b)) & mask, b, s);
    f[k] = gamma_field(c, l[k]);
    if (k >= ge) {
      f[k] = 0u;
      l[k] = 0;
    }
    tot += l[k];
  }
  return tot;
}

template <int G>
__global__ __launch_bounds__(64 * kWaves) void k_elias_count(
    int64_t n, int64_t nb, int d, int b, int s,
    const uint32_t* __restrict__ codes, uint64_t* __restrict__ off) {
  __shared__ uint32_t cnt[kChunk];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t j0 = (int64_t)blockIdx.x * kChunk;
  for (int t = wave; t < kChunk; t += kWaves) {
    const int64_t j = j0 + t;
    uint32_t bits = 0;
    if (j < nb) {
      const int64_t base = j * d;
      const int nj = (int)((n - base) < d ? (n - base) : d);
      for (int seg = 0; seg < nj; seg += 64 * G) {
        const int i0 = seg + lane * G;
        const int ge = max(0, min(G, nj - i0));
        uint32_t f[G];
        int l[G];
        bits += (uint32_t)lane_fields<G>(codes, base + i0, ge, b, s, f, l);
      }
      bits = (uint32_t)group_sum_i<64>((int)bits);
    }
    if (lane == 0) cnt[t] = (bits + 31u) >> 5;
  }
  __syncthreads();
  if (wave == 0) {
    const uint32_t v = wave_incl_scan(cnt[lane]);
    const int64_t j = j0 + lane;
    if (j < nb) off[j + 1] = v;
  }
}

__global__ __launch_bounds__(kScan) void k_elias_scan(int64_t nb,
                                                      uint64_t* __restrict__ off) {
  __shared__ uint64_t part[2][kScan];
  const int t = threadIdx.x;
  const int64_t nc = (nb + kChunk - 1) / kChunk;
  const int64_t per = (nc + kScan - 1) / kScan;
  const int64_t c0 = (int64_t)t * per, c1 = min(nc, c0 + per);
  uint64_t sum = 0;
  for (int64_t c = c0; c < c1; ++c) sum += off[min((c + 1) * kChunk, nb)];
  part[0][t] = sum;
  __syncthreads();
  int src = 0;
  for (int o = 1; o < kScan; o <<= 1) {  // inclusive scan, double-buffered
    const uint64_t v = part[src][t] + (t >= o ? part[src][t - o] : 0ull);
    part[src ^ 1][t] = v;
    src ^= 1;
    __syncthreads();
  }
  uint64_t run = part[src][t] - sum;  // exclusive prefix of this thread
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t i = min((c + 1) * kChunk, nb);
    run += off[i];
    off[i] = run;
  }
  if (t == 0) off[0] = 0;
}

template <int G>
__global__ __launch_bounds__(64 * kWaves) void k_elias_write(
    int64_t n, int64_t nb, int d, int b, int s, int64_t cap,
    const uint32_t* __restrict__ codes, uint64_t* __restrict__ off,
    uint32_t* __restrict__ words) {
  // worst segment: 64 G codes of 16 bits, shifted by up to 31 carried bits
  constexpr int kWin = 32 * G + 2;
  __shared__ uint32_t win_all[kWaves][kWin];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t* win = win_all[wave];
  const int64_t j = (int64_t)blockIdx.x * kWaves + wave;
  const bool live = j < nb;
  int64_t start = 0;
  int nj = 0;
  if (live) {
    const int64_t cs = j - j % kChunk;
    const uint64_t oj = off[j];
    start = (int64_t)(j == cs ? oj : off[cs] + oj);
    nj = (int)((n - j * d) < d ? (n - j * d) : d);
  }
  if (live && j % kChunk != 0 && lane == 0) off[j] = (uint64_t)start;
  uint32_t carry = 0;  // low bits of the record's current partial word
  int pos = 0;         // record bits written so far
  const int nseg = d / (64 * G);  // the same for every wave of the block
  for (int sg = 0; sg < nseg; ++sg) {
    const int i0 = sg * 64 * G + lane * G;
    const int ge = max(0, min(G, nj - i0));
    uint32_t f[G];
    int l[G];
    const int tot = lane_fields<G>(codes, j * d + i0, ge, b, s, f, l);
    const int incl = (int)wave_incl_scan((uint32_t)tot);
    const int seg_bits = __shfl(incl, 63, 64);
    const int p0 = pos & 31;
    const int nw = (p0 + seg_bits + 31) >> 5;
    for (int w = lane; w < nw; w += 64) win[w] = w == 0 ? carry : 0u;
    __syncthreads();
    if (tot > 0) {
      const int at = p0 + incl - tot;
      int wi = at >> 5, ab = at & 31;
      uint64_t acc = 0;
#pragma unroll
      for (int k = 0; k < G; ++k) {
        acc |= (uint64_t)f[k] << ab;
        ab += l[k];
        if (ab >= 32) {
          atomicOr(&win[wi], (uint32_t)acc);
          acc >>= 32;
          ab -= 32;
          ++wi;
        }
      }
      if (ab > 0) atomicOr(&win[wi], (uint32_t)acc);
    }
    __syncthreads();
    const int full = (p0 + seg_bits) >> 5;
    const int64_t w0 = start + (pos >> 5);
    // cap (the worst-case stream length) is a guard only: records sized by
    // the count pass never reach it
    if (live)
      for (int w = lane; w < full; w += 64)
        if (w0 + w < cap) words[w0 + w] = win[w];
    carry = ((p0 + seg_bits) & 31) ? win[full] : 0u;
    pos += seg_bits;
    __syncthreads();
  }
  if (live && lane == 0 && (pos & 31) && start + (pos >> 5) < cap)
    words[start + (pos >> 5)] = carry;
}

__global__ __launch_bounds__(256) void k_elias_decode(
    int64_t n, int64_t nb, int d, int b, int64_t n_words,
    const uint64_t* __restrict__ off, const uint32_t* __restrict__ words,
    uint32_t* __restrict__ codes) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= nb) return;
  const uint64_t lim = (uint64_t)n_words;  // >= 1
  const uint64_t a = min(off[j], lim);
  const uint64_t e = min(max(off[j + 1], a), lim);
  // ring slot r holds stream word widx + r; loads are unconditional (index
  // clamped into the stream) and words past the record are zeroed when used,
  // so a slot's load is only waited for when the slot is consumed
  uint32_t ring[kLook];
#pragma unroll
  for (int k = 0; k < kLook; ++k) ring[k] = words[min(a + k, lim - 1)];
  uint64_t widx = a;
  uint64_t win = 0;
  int avail = 0;
  const uint32_t mask = (1u << b) - 1u;
  uint64_t ob = 0;
  int obits = 0;
  int64_t ow = j * (d / 32) * b;  // the bucket's first code word
  const int nj = (int)((n - j * d) < d ? (n - j * d) : d);
  int i = 0;
  while (i < nj) {
#pragma unroll
    for (int r = 0; r < kLook; ++r) {
      win |= (uint64_t)(widx < e ? ring[r] : 0u) << avail;
      avail += 32;
      ring[r] = words[min(widx + kLook, lim - 1)];
      ++widx;
      for (; avail > 32 && i < nj; ++i) {
        // a zero run longer than 15 only occurs in a corrupt stream
        const int L = __builtin_ctzll(win | (1ull << 15));
        const uint32_t dig = (uint32_t)(win >> L) & ((2u << L) - 1u);
        const uint32_t m = __brev(dig) >> (31 - L);
        const bool neg = (win >> (2 * L + 1)) & 1ull;
        const int mag = (int)m - 1;
        const int c = L == 0 ? 0 : (neg ? -mag : mag);
        const int len = L == 0 ? 1 : 2 * L + 2;
        win >>= len;
        avail -= len;
        ob |= (uint64_t)((uint32_t)c & mask) << obits;
        obits += b;
        if (obits >= 32) {
          codes[ow++] = (uint32_t)ob;
          ob >>= 32;
          obits -= 32;
        }
      }
    }
  }
  if (obits > 0) codes[ow] = (uint32_t)ob;
}

}  // namespace

int64_t elias_max_words(const LaunchDesc& L, int64_t n);

namespace {

template <int G>
int encode_g(const LaunchDesc& L, int64_t n, const uint32_t* codes,
             uint64_t* off, uint32_t* words, hipStream_t st) {
  const int64_t nb = (n + L.d - 1) / L.d;
  const int64_t nblk = (nb + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(k_elias_count<G>, dim3((unsigned)nblk), dim3(64 * kWaves), 0,
                     st, n, nb, L.d, L.bits, L.s, codes, off);
  hipLaunchKernelGGL(k_elias_scan, dim3(1), dim3(kScan), 0, st, nb, off);
  hipLaunchKernelGGL(k_elias_write<G>, dim3((unsigned)((nb + kWaves - 1) / kWaves)),
                     dim3(64 * kWaves), 0, st, n, nb, L.d, L.bits, L.s,
                     elias_max_words(L, n), codes, off, words);
  return (int)hipGetLastError();
}

}  // namespace

int64_t elias_max_words(const LaunchDesc& L, int64_t n) {
  const uint32_t m = (uint32_t)L.s + 1u;
  int fl = 0;
  while ((m >> (fl + 1)) != 0) ++fl;
  const int64_t worst = 2 * fl + 2;  // bits of a code with |c| = s
  const int64_t nb = (n + L.d - 1) / L.d;
  const int64_t last = n - (nb - 1) * L.d;
  return (nb - 1) * ((L.d * worst) / 32) + (last * worst + 31) / 32;
}

int launch_elias_encode(const LaunchDesc& L, int64_t n, const uint8_t* codes,
                        uint64_t* off, uint32_t* words, hipStream_t st) {
  const uint32_t* c = reinterpret_cast<const uint32_t*>(codes);
  switch (L.d >= 512 ? 8 : L.d / 64) {
    case 1: return encode_g<1>(L, n, c, off, words, st);
    case 2: return encode_g<2>(L, n, c, off, words, st);
    case 4: return encode_g<4>(L, n, c, off, words, st);
    default: return encode_g<8>(L, n, c, off, words, st);
  }
}

int launch_elias_decode(const LaunchDesc& L, int64_t n, const uint64_t* off,
                        const uint32_t* words, int64_t n_words, uint8_t* codes,
                        hipStream_t st) {
  const int64_t nb = (n + L.d - 1) / L.d;
  hipLaunchKernelGGL(k_elias_decode, dim3((unsigned)((nb + 255) / 256)), dim3(256),
                     0, st, n, nb, L.d, L.bits, n_words, off, words,
                     reinterpret_cast<uint32_t*>(codes));
  return (int)hipGetLastError();
}

}  // namespace gq
