// elias.hip — Elias gamma coding of uniform-scheme codes, the lossless step
// QSGD applies to its quantized integers ("Gradient Quantization" glossary,
// QSGD paragraph).  Code c becomes gamma(m), m = |c| + 1 (floor(log2 m)
// zeros, then the digits of m from the most significant), then a sign bit
// (1 = negative) when c != 0.  Each bucket's record starts on a 32-bit word;
// off[j] is the first word of record j and off[nb] the stream's length.
//
// Encode: three launches, no scratch memory.
//   1. k_elias_count: a block owns kChunk consecutive buckets, a wave
//      kPerWave of them (their loads issued together).  Each bucket's word
//      count, then the chunk's inclusive scan: off[j + 1] = words of the
//      chunk's buckets up to j.
//   2. k_elias_scan: one block turns the chunk totals (each sits at its
//      chunk's last entry) into global inclusive sums in place; off[0] = 0.
//   3. k_elias_write: one wave (and block) per bucket.  Record j starts at
//      off[chunk start] + off[j] (entries at chunk starts are final after
//      step 2; the wave writes the final off[j] back).  Per segment of 64 G
//      elements, lane l takes G consecutive codes, a wave scan of their bit
//      counts places them, each lane ORs its bits into the wave's LDS window
//      32 at a time, and the segment's whole words go out; the last partial
//      word carries into the next segment.
// Decode: one lane per bucket parses its record serially from a 64-bit
// window kept above 32 bits.  A step looks the window's next kLutBits bits
// up in an LDS table of the whole codewords they hold (codes already in the
// b-bit output format) and takes them all; a longer codeword is decoded
// directly.  The window is fed from an LDS row of the lane's next kRow
// stream words, staged with kRow independent loads and restaged for the
// whole wave when some lane has used its row.
#include "common.hpp"

namespace gq {
namespace {

constexpr int kChunk = 64;       // buckets per block in the count pass
constexpr int kCountWaves = 16;  // waves per block of the count pass
constexpr int kPerWave = kChunk / kCountWaves;
constexpr int kScan = 1024;   // threads of the one-block scan
constexpr int kDecWaves = 1;  // waves per block of the decoder
constexpr int kRow = 32;      // decode: stream words staged per lane
constexpr int kLutBits = 10;  // decode: stream bits that index the table
constexpr int kLut = 1 << kLutBits;

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

// Inclusive prefix sum over the wave: shifts of 1, 2, 4, 8 lanes inside
// each row of 16 (lanes shifted in from outside the row read 0), then each
// row's total broadcast into the rows above it (lane 15 into rows 1 and 3,
// lane 31 into rows 2 and 3).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false); // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false); // row_bcast:31
  return (uint32_t)x;
}

// Per-code tables for code widths b <= 4 (raw b-bit code r, clamped to
// [-s, s]): len = bits [4r, 4r + 4) of len_t; field = byte r of
// field_t[r / 8] (gamma codewords of |c| <= 7 fit in 8 bits).  b = 8 uses
// gamma_field directly.
struct GammaTab {
  uint64_t len_t;
  uint64_t field_t[2];
};

// The lane's G codes of a segment, starting at element e0 (ge of them live).
template <int G>
__device__ __forceinline__ uint64_t lane_codes(const uint32_t* __restrict__ codes,
                                               int64_t e0, int ge, int b) {
  return ge > 0 ? stream_bits(codes, e0 * b, ge * b) : 0ull;
}

// Gamma fields and lengths of the lane's codes; returns their total bits.
template <int G>
__device__ __forceinline__ int lane_fields(uint64_t x, int ge, int b, int s,
                                           const GammaTab& T, uint32_t (&f)[G],
                                           int (&l)[G]) {
  const uint32_t mask = (1u << b) - 1u;
  int tot = 0;
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const uint32_t r = (uint32_t)(x >> (k * b)) & mask;
    if (b <= 4) {
      l[k] = (int)((T.len_t >> (4 * r)) & 15u);
      f[k] = (uint32_t)((T.field_t[r >> 3] >> (8 * (r & 7))) & 255u);
    } else {
      f[k] = gamma_field(sext_clamp(r, b, s), l[k]);
    }
    if (k >= ge) {
      f[k] = 0u;
      l[k] = 0;
    }
    tot += l[k];
  }
  return tot;
}

// Total gamma bits of the lane's codes (lengths only).
template <int G>
__device__ __forceinline__ int lane_bits(uint64_t x, int ge, int b, int s,
                                         uint64_t len_t) {
  const uint32_t mask = (1u << b) - 1u;
  int tot = 0;
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const uint32_t r = (uint32_t)(x >> (k * b)) & mask;
    int len;
    if (b <= 4) {
      len = (int)((len_t >> (4 * r)) & 15u);
    } else {
      const int c = sext_clamp(r, b, s);
      const int a = c < 0 ? -c : c;
      len = c == 0 ? 1 : 2 * (31 - __clz(a + 1)) + 2;
    }
    tot += k < ge ? len : 0;
  }
  return tot;
}

// kCountWaves waves per block, kPerWave buckets per wave: the loads of a
// wave's buckets are issued together.  A grid smaller than the number of
// chunks strides over them.
template <int G>
__global__ __launch_bounds__(64 * kCountWaves) void k_elias_count(
    int64_t n, int64_t nb, int d, int b, int s, uint64_t len_t,
    const uint32_t* __restrict__ codes, uint64_t* __restrict__ off) {
  __shared__ uint32_t cnt[kChunk];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nc = (nb + kChunk - 1) / kChunk;
  for (int64_t chunk = blockIdx.x; chunk < nc; chunk += gridDim.x) {
    const int64_t j0 = chunk * kChunk + wave * kPerWave;
    int nj[kPerWave];
#pragma unroll
    for (int t = 0; t < kPerWave; ++t) {
      const int64_t r = n - (j0 + t) * d;
      nj[t] = j0 + t < nb ? (int)(r < d ? r : d) : 0;
    }
    int bits[kPerWave] = {};
    const int nseg = d / (64 * G);
    for (int sg = 0; sg < nseg; ++sg) {
      const int i0 = sg * 64 * G + lane * G;
      uint64_t x[kPerWave];
      int ge[kPerWave];
#pragma unroll
      for (int t = 0; t < kPerWave; ++t) {
        ge[t] = max(0, min(G, nj[t] - i0));
        x[t] = lane_codes<G>(codes, (j0 + t) * d + i0, ge[t], b);
      }
#pragma unroll
      for (int t = 0; t < kPerWave; ++t) bits[t] += lane_bits<G>(x[t], ge[t], b, s, len_t);
    }
#pragma unroll
    for (int t = 0; t < kPerWave; ++t) {
      const uint32_t tb = (uint32_t)group_sum_i<64>(bits[t]);
      if (lane == 0) cnt[wave * kPerWave + t] = (tb + 31u) >> 5;
    }
    __syncthreads();
    if (wave == 0) {
      const uint32_t v = wave_incl_scan(cnt[lane]);
      const int64_t j = chunk * kChunk + lane;
      if (j < nb) off[j + 1] = v;
    }
    __syncthreads();  // cnt is reused by the next chunk
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
#pragma unroll 8
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
__global__ __launch_bounds__(64) void k_elias_write(
    int64_t n, int64_t nb, int d, int b, int s, int64_t cap, GammaTab T,
    const uint32_t* __restrict__ codes, uint64_t* __restrict__ off,
    uint32_t* __restrict__ words) {
  // worst segment: 64 G codes of 16 bits, shifted by up to 31 carried bits
  constexpr int kWin = 32 * G + 2;
  __shared__ uint32_t win[kWin];
  const int lane = threadIdx.x;
  // one bucket per block; a grid smaller than nb strides (uniform per block)
  for (int64_t j = blockIdx.x; j < nb; j += gridDim.x) {
    const int64_t cs = j - j % kChunk;  // the chunk's first bucket
    const uint64_t oj = off[j];
    const int64_t start = (int64_t)(j == cs ? oj : off[cs] + oj);
    const int nj = (int)((n - j * d) < d ? (n - j * d) : d);
    if (j != cs && lane == 0) off[j] = (uint64_t)start;
    uint32_t carry = 0;  // low bits of the record's current partial word
    int pos = 0;         // record bits written so far
    const int nseg = d / (64 * G);
    for (int sg = 0; sg < nseg; ++sg) {
      const int i0 = sg * 64 * G + lane * G;
      const int ge = max(0, min(G, nj - i0));
      uint32_t f[G];
      int l[G];
      const int tot =
          lane_fields<G>(lane_codes<G>(codes, j * d + i0, ge, b), ge, b, s, T, f, l);
      const int incl = (int)wave_incl_scan((uint32_t)tot);
      const int seg_bits = __builtin_amdgcn_readlane(incl, 63);
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
      for (int w = lane; w < full; w += 64)
        if (w0 + w < cap) words[w0 + w] = win[w];
      carry = ((p0 + seg_bits) & 31) ? win[full] : 0u;
      pos += seg_bits;
      __syncthreads();
    }
    if (lane == 0 && (pos & 31) && start + (pos >> 5) < cap)
      words[start + (pos >> 5)] = carry;
    __syncthreads();  // the window is reused by the next bucket
  }
}

// Decode table entry for the next kLutBits stream bits v: the complete
// codewords they hold from bit 0, as codes packed b bits each (at most 32
// bits of codes), their count k and their total length.  k = 0: the first
// codeword is longer than kLutBits (or v holds no whole codeword).
constexpr uint64_t lut_entry(uint32_t v, int b) {
  const uint32_t mask = (1u << b) - 1u;
  uint32_t out = 0;
  int k = 0, pos = 0;
  for (;;) {
    const uint32_t rest = v >> pos;
    if (rest == 0) break;  // only zeros left: no codeword ends here
    int L = 0;
    while (((rest >> L) & 1u) == 0) ++L;
    const int len = L == 0 ? 1 : 2 * L + 2;
    if (pos + len > kLutBits || (k + 1) * b > 32) break;
    uint32_t m = 0;  // the L + 1 digits, most significant first
    for (int t = 0; t <= L; ++t) m = (m << 1) | ((rest >> (L + t)) & 1u);
    int c = (int)m - 1;
    if (L > 0 && ((rest >> (2 * L + 1)) & 1u)) c = -c;
    out |= ((uint32_t)c & mask) << (k * b);
    ++k;
    pos += len;
  }
  return (uint64_t)out | ((uint64_t)k << 32) | ((uint64_t)pos << 40);
}

// The decode tables of the four code widths, built at compile time.
struct DecodeLut {
  uint64_t e[kLut];
  constexpr explicit DecodeLut(int b) : e{} {
    for (uint32_t v = 0; v < (uint32_t)kLut; ++v) e[v] = lut_entry(v, b);
  }
};
__device__ constexpr DecodeLut kLut2{2};
__device__ constexpr DecodeLut kLut3{3};
__device__ constexpr DecodeLut kLut4{4};
__device__ constexpr DecodeLut kLut8{8};

__global__ __launch_bounds__(64 * kDecWaves) void k_elias_decode(
    int64_t n, int64_t nb, int d, int b, int64_t n_words,
    const uint64_t* __restrict__ off, const uint32_t* __restrict__ words,
    uint32_t* __restrict__ codes) {
  __shared__ uint64_t lut[kLut];
  // each lane's next kRow stream words (padded rows: no bank conflicts when
  // every lane stages word k at once)
  __shared__ uint32_t rows_all[kDecWaves][64][kRow + 1];
  const uint64_t* src =
      b == 2 ? kLut2.e : (b == 3 ? kLut3.e : (b == 4 ? kLut4.e : kLut8.e));
  for (int t = threadIdx.x; t < kLut; t += 64 * kDecWaves) lut[t] = src[t];
  __syncthreads();  // the table
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // one lane per bucket; a grid smaller than nb / 64 strides (uniform per wave)
  const int64_t stride = (int64_t)gridDim.x * kDecWaves * 64;
  for (int64_t j0 = ((int64_t)blockIdx.x * kDecWaves + wave) * 64; j0 < nb; j0 += stride) {
    const int64_t j = j0 + lane;
    const bool live = j < nb;
    uint32_t* row = rows_all[wave][lane];
    const uint64_t lim = (uint64_t)n_words;  // >= 1
    uint64_t base = 0, e = 0;                // row[0] holds stream word base
    int nj = 0;
    if (live) {
      base = min(off[j], lim);
      e = min(max(off[j + 1], base), lim);
      nj = (int)((n - j * d) < d ? (n - j * d) : d);
    }
    // all kRow loads of a lane are issued before the first is used; words
    // past the record (or the readable stream) are staged as 0
    auto restage = [&]() {
      uint32_t v[kRow];
#pragma unroll
      for (int k = 0; k < kRow; ++k) v[k] = words[min(base + k, lim - 1)];
#pragma unroll
      for (int k = 0; k < kRow; ++k) row[k] = base + k < e ? v[k] : 0u;
    };
    restage();
    int rp = 0;  // next row word for the window
    uint64_t win = 0;
    int avail = 0;
    const uint32_t mask = (1u << b) - 1u;
    uint64_t ob = 0;
    int obits = 0;
    int64_t ow = j * (int64_t)(d / 32) * b;  // the bucket's first code word
    const int64_t ow_end = ow + (((int64_t)nj * b + 31) >> 5);
    int i = 0;  // codes decoded
    // every step of a lane takes at least one codeword (refills: at most one
    // row word per step), so the loop ends within d steps
    while (__any(i < nj)) {
      if (__any(i < nj && avail <= 32 && rp >= kRow)) {
        base += (uint64_t)rp;
        rp = 0;
        restage();
      }
      if (i < nj) {
        if (avail <= 32) {
          win |= (uint64_t)row[rp] << avail;
          avail += 32;
          ++rp;
        }
        const uint64_t ent = lut[(uint32_t)win & (kLut - 1)];
        uint32_t out = (uint32_t)ent;
        int k = (int)(ent >> 32) & 255;
        int len = (int)(ent >> 40) & 255;
        if (k == 0) {
          // one long codeword; a zero run past 15 only occurs in a corrupt stream
          const int L = __builtin_ctzll(win | (1ull << 15));
          const uint32_t dig = (uint32_t)(win >> L) & ((2u << L) - 1u);
          const int mag = (int)(__brev(dig) >> (31 - L)) - 1;
          const bool neg = (win >> (2 * L + 1)) & 1ull;
          out = (uint32_t)(L == 0 ? 0 : (neg ? -mag : mag)) & mask;
          k = 1;
          len = L == 0 ? 1 : 2 * L + 2;
        }
        if (k > nj - i) {  // codes past the bucket's last element are dropped
          k = nj - i;
          out &= (1u << (k * b)) - 1u;
        }
        win >>= len;
        avail -= len;
        i += k;
        ob |= (uint64_t)out << obits;
        obits += k * b;
        if (obits >= 32) {
          if (ow < ow_end) codes[ow] = (uint32_t)ob;
          ++ow;
          ob >>= 32;
          obits -= 32;
        }
      }
    }
    if (obits > 0 && ow < ow_end) codes[ow] = (uint32_t)ob;
  }
}

}  // namespace

int64_t elias_max_words(const LaunchDesc& L, int64_t n);

namespace {

GammaTab gamma_tab(int b, int s) {
  GammaTab T{0, {0, 0}};
  if (b > 4) return T;
  for (uint32_t r = 0; r < (1u << b); ++r) {
    int c = (int)(r << (32 - b)) >> (32 - b);
    c = c < -s ? -s : (c > s ? s : c);
    const uint32_t m = (uint32_t)(c < 0 ? -c : c) + 1u;
    int L = 0;
    while ((m >> (L + 1)) != 0) ++L;
    // L zeros, the L + 1 digits of m from the most significant, the sign
    uint32_t f = 0;
    int t = L;
    for (int k = L; k >= 0; --k, ++t) f |= ((m >> k) & 1u) << t;
    if (c != 0) f |= (c < 0 ? 1u : 0u) << t++;
    T.len_t |= (uint64_t)t << (4 * r);
    T.field_t[r >> 3] |= (uint64_t)f << (8 * (r & 7));
  }
  return T;
}

template <int G>
int encode_g(const LaunchDesc& L, int64_t n, const uint32_t* codes,
             uint64_t* off, uint32_t* words, hipStream_t st) {
  const int64_t nb = (n + L.d - 1) / L.d;
  // grids stay below 2^32 work-items (a dispatch's limit); larger inputs stride
  const int64_t nc = (nb + kChunk - 1) / kChunk;
  const int64_t nblk = nc < (int64_t(1) << 20) ? nc : (int64_t(1) << 20);
  const GammaTab T = gamma_tab(L.bits, L.s);
  hipLaunchKernelGGL(k_elias_count<G>, dim3((unsigned)nblk), dim3(64 * kCountWaves), 0,
                     st, n, nb, L.d, L.bits, L.s, T.len_t, codes, off);
  hipLaunchKernelGGL(k_elias_scan, dim3(1), dim3(kScan), 0, st, nb, off);
  const int64_t wgrid = nb < (int64_t(1) << 24) ? nb : (int64_t(1) << 24);
  hipLaunchKernelGGL(k_elias_write<G>, dim3((unsigned)wgrid), dim3(64), 0, st, n, nb,
                     L.d, L.bits, L.s, elias_max_words(L, n), T, codes, off, words);
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
  const int64_t per_block = 64 * kDecWaves;
  int64_t grid = (nb + per_block - 1) / per_block;
  grid = grid < (int64_t(1) << 24) ? grid : (int64_t(1) << 24);
  hipLaunchKernelGGL(k_elias_decode, dim3((unsigned)grid),
                     dim3(64 * kDecWaves),
                     0, st, n, nb, L.d, L.bits, n_words, off, words,
                     reinterpret_cast<uint32_t*>(codes));
  return (int)hipGetLastError();
}

}  // namespace gq
