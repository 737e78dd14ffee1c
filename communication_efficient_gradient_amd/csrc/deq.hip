// deq.hip — decompress side: unpack, dequantize and accumulate W payloads
// into an fp32 average ("gradient quantization for communication" glossary,
// §How Gradient Quantization Works: dequantize, then aggregate), and the
// standalone residual update of error feedback ("Gradient Quantization"
// glossary, error-feedback paragraph).
//
// Output-stationary and lane-contiguous: a thread owns kV float4 groups of
// the output, group f covering elements 4f .. 4f+3 (one bucket, since d is a
// multiple of 4), and neighbouring lanes own neighbouring groups, so every
// 128-bit store and load of a wave covers 1 KiB of consecutive memory.  For
// the uniform scheme the per-bucket step M/s is divided out once per
// (payload, bucket) of a block and read from LDS.  The
// codes of a group are 4*BITS consecutive stream bits: one byte load (1, 2
// bits), two (3 bits), a 16-bit (4 bits) or a 32-bit (8 bits) load, again
// consecutive across lanes.  Payloads are summed in fp32 into two
// accumulators (even and odd payloads), so a sum of W terms is at most
// ceil(W/2)+1 additions deep.  The fp32 streams (aggregate, gradient,
// residual) use nontemporal 128-bit accesses.
#include "common.hpp"

namespace gq {
namespace {

constexpr int kThreads = 256;
constexpr int kV = 2;                       // float4 groups per thread
constexpr int kGroupsPerBlock = kThreads * kV;

// The 4*BITS code bits of group f (elements 4f..4f+3), element 4f in the
// lowest bits.  `full` groups lie wholly inside the stream; the last,
// partial group reads byte by byte up to code_bytes.
template <int BITS>
__device__ __forceinline__ uint32_t load_codes4(const uint8_t* __restrict__ c,
                                                int64_t f, bool full,
                                                int64_t code_bytes) {
  const int64_t bit0 = (int64_t)4 * BITS * f;
  const int64_t byte0 = bit0 >> 3;
  const int sh = (int)(bit0 & 7);
  if (full) {
    if constexpr (BITS == 1) return ((uint32_t)c[byte0] >> sh) & 0xFu;
    if constexpr (BITS == 2) return (uint32_t)c[byte0];
    if constexpr (BITS == 3)
      return (((uint32_t)c[byte0] | ((uint32_t)c[byte0 + 1] << 8)) >> sh) & 0xFFFu;
    if constexpr (BITS == 4) return (uint32_t)*reinterpret_cast<const uint16_t*>(c + byte0);
    if constexpr (BITS == 8) return *reinterpret_cast<const uint32_t*>(c + byte0);
  }
  // bytes a group can touch: its 4*BITS bits start at bit 0 or 4 of a byte
  uint32_t w = 0u;
  constexpr int kBytes = BITS == 8 ? 4 : (4 * BITS + 4 + 7) / 8;
#pragma unroll
  for (int b = 0; b < kBytes; ++b)
    if (byte0 + b < code_bytes) w |= (uint32_t)c[byte0 + b] << (8 * b);
  w >>= sh;
  return BITS == 8 ? w : (w & ((1u << (4 * BITS)) - 1u));
}

// Dense packing (BITS = 0): field width, alphabet size, A^4 and the
// reciprocals for the digit split.
struct DenseCfg {
  int W;
  uint32_t A, A4;
  DenseRecip r;
};

// The codes of group f: BITS-bit fields (element 4f in the low bits) or,
// dense, four 8-bit digits (digit k in bits 8k .. 8k+7).
template <int BITS>
__device__ __forceinline__ uint32_t load_group(const uint8_t* __restrict__ c,
                                               int64_t f, bool full,
                                               int64_t code_bytes,
                                               const DenseCfg& dc) {
  if constexpr (BITS == 0)
    return load_dense4(c, f, dc.W, dc.A, dc.A4, dc.r, code_bytes);
  else
    return load_codes4<BITS>(c, f, full, code_bytes);
}

// Code value k of a loaded group: the signed integer -s..s for the uniform
// scheme (two's complement, or dense digit - s), the level index otherwise.
template <int SCHEME, int BITS>
__device__ __forceinline__ int code_value(uint32_t w, int k, int s) {
  if constexpr (BITS == 0) {
    const int digit = (int)((w >> (8 * k)) & 0xFFu);
    return SCHEME == UNIFORM ? digit - s : digit;
  } else {
    const uint32_t u = (w >> (BITS * k)) & ((1u << BITS) - 1u);
    if constexpr (SCHEME == UNIFORM) {
      const uint32_t m = 1u << (BITS - 1);
      return (int)((u ^ m) - m);  // sign-extend
    } else {
      return (int)u;
    }
  }
}

// Dequantized values of one group of one payload.
template <int SCHEME, int BITS>
__device__ __forceinline__ float4 dequant4(uint32_t w,
                                           const float* __restrict__ meta,
                                           int64_t bucket, int s, int L) {
  float x[4];
  if constexpr (SCHEME == UNIFORM) {
    const float delta = meta[bucket] / (float)s;
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = (float)code_value<SCHEME, BITS>(w, k, s) * delta;
  } else if constexpr (SCHEME == BIN_SIGN || SCHEME == BIN_OPT) {
    const float a = meta[2 * bucket + 0], b = meta[2 * bucket + 1];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = ((w >> k) & 1u) ? b : a;
  } else {
    // codes past the level table (never written by the quantizer) are
    // clamped so that no read leaves the bucket's meta row
    const float* lv = meta + bucket * L;
    const uint32_t top = (uint32_t)(L - 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t c = (uint32_t)code_value<SCHEME, BITS>(w, k, s);
      x[k] = lv[c < top ? c : top];
    }
  }
  return make_float4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

template <int SCHEME, int BITS, int NB>
__global__ __launch_bounds__(kThreads) void k_deq_acc(
    int64_t n, int dsh, int s, int L, int W, PayloadPtrs pp, float alpha,
    float beta, float* __restrict__ out, int64_t code_bytes, DenseCfg dc) {
  // The block's tile is kGroupsPerBlock consecutive groups; pass v of the
  // block covers the kThreads groups [tile + kThreads v, tile + kThreads
  // (v + 1)), thread t taking group tile + kThreads v + t.
  const int64_t ngroups = (n + 3) >> 2;
  const int64_t tile = (int64_t)blockIdx.x * kGroupsPerBlock;
  const int64_t f0 = tile + threadIdx.x;
  constexpr int kStride = kThreads;  // groups between a thread's v and v+1

  // Code loads of NB payloads at once (NB = 1, 2 or 4), all issued before
  // any use, together with the loads of the bucket's scale (uniform scheme
  // without the LDS table) or two levels (two-level schemes), which do not
  // depend on the codes.  ORQ levels are looked up by code afterwards.
  constexpr bool TABLE = NB == 4;
  constexpr int MK = SCHEME == UNIFORM ? (TABLE ? 0 : 1)
                                       : (SCHEME == ORQ ? 0 : 2);
  uint32_t cw[NB][kV];
  float mv[NB][kV][MK > 0 ? MK : 1];
  auto load_batch = [&](int p0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int p = p0 + j;
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        const int64_t f = f0 + kStride * v;
        const bool live = p < W && f < ngroups;
        cw[j][v] = live ? load_group<BITS>(pp.codes[p < W ? p : 0], f,
                                           4 * f + 4 <= n, code_bytes, dc)
                        : 0u;
        if constexpr (MK > 0) {
          const float* m = pp.meta[p < W ? p : 0] + MK * ((4 * f) >> dsh);
#pragma unroll
          for (int t = 0; t < MK; ++t) mv[j][v][t] = live ? m[t] : 0.f;
        }
      }
    }
  };
  load_batch(0);

  // Uniform scheme with TABLE (NB = 4, W >= 3): the step M/s of every (payload,
  // bucket) the tile touches, one correctly rounded division each, shared
  // through LDS (built while the first code loads are in flight).  For one
  // or two payloads each group divides for itself: the barrier would cost
  // more than the divisions it saves.
  __shared__ float delta_tab[TABLE ? kMaxPayloads * (kGroupsPerBlock * 4 / 64 + 1) : 1];
  const int64_t b0 = (4 * tile) >> dsh;
  int nbk = 0;
  if constexpr (SCHEME == UNIFORM && TABLE) {
    const int64_t last = (4 * (tile + kGroupsPerBlock) - 1) >> dsh;
    const int64_t nb = (n + ((int64_t)1 << dsh) - 1) >> dsh;
    nbk = (int)(last - b0 + 1);
    for (int t = threadIdx.x; t < W * nbk; t += kThreads) {
      const int p = t / nbk, j = t % nbk;
      const int64_t bucket = b0 + j;
      delta_tab[t] = bucket < nb ? pp.meta[p][bucket] / (float)s : 0.f;
    }
    __syncthreads();
  }
  auto deq = [&](int j, int v, int p, int64_t f) -> float4 {
    const uint32_t w = cw[j][v];
    const int64_t bucket = (4 * f) >> dsh;
    float x[4];
    if constexpr (SCHEME == UNIFORM) {
      float delta;
      if constexpr (TABLE) delta = delta_tab[p * nbk + (int)(bucket - b0)];
      else delta = mv[j][v][0] / (float)s;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        x[k] = (float)code_value<SCHEME, BITS>(w, k, s) * delta;
    } else if constexpr (SCHEME == BIN_SIGN || SCHEME == BIN_OPT) {
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = ((w >> k) & 1u) ? mv[j][v][1] : mv[j][v][0];
    } else {
      return dequant4<SCHEME, BITS>(w, pp.meta[p], bucket, s, L);
    }
    return make_float4(x[0], x[1], x[2], x[3]);
  };

  // Payloads 0 and 1 initialise the two accumulators (a copy, so a single
  // payload is reproduced bit for bit); later even / odd payloads add into
  // acc0 / acc1 in payload order.
  float4 acc0[kV], acc1[kV];
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    acc0[v] = make_float4(0.f, 0.f, 0.f, 0.f);
    acc1[v] = acc0[v];
  }
  for (int p0 = 0; p0 < W; p0 += NB) {
    if (p0 > 0) load_batch(p0);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int p = p0 + j;
      if (p >= W) break;
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        const int64_t f = f0 + kStride * v;
        if (f >= ngroups) continue;
        const float4 x = deq(j, v, p, f);
        if (p == 0) acc0[v] = x;
        else if (p == 1) acc1[v] = x;
        else if (p & 1) acc1[v] = add4(acc1[v], x);
        else acc0[v] = add4(acc0[v], x);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    const int64_t f = f0 + kStride * v;
    if (f >= ngroups) continue;
    float4 a = W > 1 ? add4(acc0[v], acc1[v]) : acc0[v];
    float4 r = make_float4(alpha * a.x, alpha * a.y, alpha * a.z, alpha * a.w);
    float* o = out + 4 * f;
    if (4 * f + 4 <= n) {
      if (beta != 0.f) {
        const float4 old = load4_nt(o);
        r.x = r.x + beta * old.x;
        r.y = r.y + beta * old.y;
        r.z = r.z + beta * old.z;
        r.w = r.w + beta * old.w;
      }
      store4_nt(o, r);
    } else {
      const int rem = (int)(n - 4 * f);
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        if (k < rem) {
          float rk = comp(r, k);
          if (beta != 0.f) rk = rk + beta * o[k];
          o[k] = rk;
        }
      }
    }
  }
}

// Wide code loads for 4- and 8-bit codes.  A wave owns a run of kWideRun =
// 256 consecutive groups (1024 elements); a payload's codes for the run are
// one contiguous block of 128*BITS bytes (1 KiB of INT8 codes), loaded as one
// 2*BITS-byte vector per lane (128-bit for 8-bit codes) instead of one 4*BITS-
// bit word per group, so a wave keeps 4x more bytes in flight per load
// instruction.  The block passes through the wave's own LDS row, from which
// lane l reads the code word of group 64v + l of the run: the output stores
// stay lane-contiguous as in k_deq_acc.  Payload batches of NB (up to 8) are
// loaded before any is used; accumulation order and arithmetic are those of
// k_deq_acc, so both kernels give the same bits.  A run that reaches past
// the last whole group loads group by group as k_deq_acc does.
constexpr int kWideKV = 4;                         // groups per lane
constexpr int kWideRun = 64 * kWideKV;             // groups per wave
constexpr int kWideBlockGroups = kThreads / 64 * kWideRun;

template <int BITS> struct WideVec;
template <> struct WideVec<8> { using T = uint4; };
template <> struct WideVec<4> { using T = uint2; };

// Nontemporal 128/64-bit code loads (NT): for payloads that together exceed
// the last-level cache, where no code is read twice.
template <int BITS>
__device__ __forceinline__ typename WideVec<BITS>::T load_wide_nt(const uint8_t* p) {
  if constexpr (BITS == 8) {
    typedef unsigned nt_u4 __attribute__((ext_vector_type(4)));
    const nt_u4 t = __builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
  } else {
    typedef unsigned nt_u2 __attribute__((ext_vector_type(2)));
    const nt_u2 t = __builtin_nontemporal_load(reinterpret_cast<const nt_u2*>(p));
    return make_uint2(t.x, t.y);
  }
}

template <int SCHEME, int BITS, int NB, bool NT>
__global__ __launch_bounds__(kThreads) void k_deq_acc_wide(
    int64_t n, int dsh, int s, int L, int W, PayloadPtrs pp, float alpha,
    float beta, float* __restrict__ out, int64_t code_bytes) {
  static_assert(BITS == 4 || BITS == 8, "wide loads are for 4- and 8-bit codes");
  using VecT = typename WideVec<BITS>::T;
  constexpr int kRunWords = kWideRun * BITS / 8;   // 32-bit words of a run's codes
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ngroups = (n + 3) >> 2;
  const int64_t tile = (int64_t)blockIdx.x * kWideBlockGroups;
  const int64_t run0 = tile + (int64_t)wave * kWideRun;
  // every group of the run is whole, so all its code bytes are in the stream
  const bool whole = 4 * (run0 + kWideRun) <= n;
  const int64_t run_byte0 = run0 * BITS / 2;       // 4*BITS bits per group

  constexpr bool TABLE = NB >= 4;
  constexpr int MK = SCHEME == UNIFORM ? (TABLE ? 0 : 1) : 0;
  // whole runs: the lane's slice of the run's codes; tail runs: the code
  // words of the lane's own groups 64v + l, packed as the slice would hold
  // them after the exchange (word v of a uint4, or half-word v of a uint2)
  VecT vec[NB];
  float mv[NB][kWideKV][MK > 0 ? MK : 1];
  auto load_batch = [&](int p0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int p = p0 + j;
      const uint8_t* c = pp.codes[p < W ? p : 0];
      if (whole) {
        const uint8_t* q = c + run_byte0 + (int64_t)lane * sizeof(VecT);
        if (p >= W) vec[j] = VecT{};
        else if constexpr (NT) vec[j] = load_wide_nt<BITS>(q);
        else vec[j] = *reinterpret_cast<const VecT*>(q);
      } else {
        uint32_t t[kWideKV];
#pragma unroll
        for (int v = 0; v < kWideKV; ++v) {
          const int64_t f = run0 + 64 * v + lane;
          t[v] = (p < W && f < ngroups)
                     ? load_codes4<BITS>(c, f, 4 * f + 4 <= n, code_bytes)
                     : 0u;
        }
        if constexpr (BITS == 8) vec[j] = make_uint4(t[0], t[1], t[2], t[3]);
        else vec[j] = make_uint2(t[0] | (t[1] << 16), t[2] | (t[3] << 16));
      }
      if constexpr (MK > 0) {
#pragma unroll
        for (int v = 0; v < kWideKV; ++v) {
          const int64_t f = run0 + 64 * v + lane;
          const bool live = p < W && f < ngroups;
          mv[j][v][0] = live ? pp.meta[p < W ? p : 0][(4 * f) >> dsh] : 0.f;
        }
      }
    }
  };
  load_batch(0);

  __shared__ float delta_tab[TABLE ? kMaxPayloads * (kWideBlockGroups * 4 / 64 + 1) : 1];
  __shared__ uint32_t xrow[kThreads / 64][kRunWords];
  const int64_t b0 = (4 * tile) >> dsh;
  int nbk = 0;
  if constexpr (SCHEME == UNIFORM && TABLE) {
    const int64_t last = (4 * (tile + kWideBlockGroups) - 1) >> dsh;
    const int64_t nb = (n + ((int64_t)1 << dsh) - 1) >> dsh;
    nbk = (int)(last - b0 + 1);
    for (int t = threadIdx.x; t < W * nbk; t += kThreads) {
      const int p = t / nbk, j = t % nbk;
      const int64_t bucket = b0 + j;
      delta_tab[t] = bucket < nb ? pp.meta[p][bucket] / (float)s : 0.f;
    }
    __syncthreads();
  }

  float4 acc0[kWideKV], acc1[kWideKV];
#pragma unroll
  for (int v = 0; v < kWideKV; ++v) {
    acc0[v] = make_float4(0.f, 0.f, 0.f, 0.f);
    acc1[v] = acc0[v];
  }
  for (int p0 = 0; p0 < W; p0 += NB) {
    if (p0 > 0) load_batch(p0);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int p = p0 + j;
      if (p >= W) break;
      uint32_t cw[kWideKV];
      if (whole) {
        // the wave's row: written by every lane, then read lane-contiguously;
        // LDS accesses of one wave execute in order, so no barrier is needed
        // between this write, the reads and the next payload's write
        reinterpret_cast<VecT*>(xrow[wave])[lane] = vec[j];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int v = 0; v < kWideKV; ++v) {
          if constexpr (BITS == 8)
            cw[v] = xrow[wave][64 * v + lane];
          else
            cw[v] = reinterpret_cast<const uint16_t*>(xrow[wave])[64 * v + lane];
        }
        __builtin_amdgcn_wave_barrier();
      } else if constexpr (BITS == 8) {
        cw[0] = vec[j].x; cw[1] = vec[j].y; cw[2] = vec[j].z; cw[3] = vec[j].w;
      } else {
        cw[0] = vec[j].x & 0xFFFFu; cw[1] = vec[j].x >> 16;
        cw[2] = vec[j].y & 0xFFFFu; cw[3] = vec[j].y >> 16;
      }
#pragma unroll
      for (int v = 0; v < kWideKV; ++v) {
        const int64_t f = run0 + 64 * v + lane;
        if (f >= ngroups) continue;
        const int64_t bucket = (4 * f) >> dsh;
        float4 x;
        if constexpr (SCHEME == UNIFORM) {
          float delta;
          if constexpr (TABLE) delta = delta_tab[p * nbk + (int)(bucket - b0)];
          else delta = mv[j][v][0] / (float)s;
          x.x = (float)code_value<SCHEME, BITS>(cw[v], 0, s) * delta;
          x.y = (float)code_value<SCHEME, BITS>(cw[v], 1, s) * delta;
          x.z = (float)code_value<SCHEME, BITS>(cw[v], 2, s) * delta;
          x.w = (float)code_value<SCHEME, BITS>(cw[v], 3, s) * delta;
        } else {
          x = dequant4<SCHEME, BITS>(cw[v], pp.meta[p], bucket, s, L);
        }
        if (p == 0) acc0[v] = x;
        else if (p == 1) acc1[v] = x;
        else if (p & 1) acc1[v] = add4(acc1[v], x);
        else acc0[v] = add4(acc0[v], x);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < kWideKV; ++v) {
    const int64_t f = run0 + 64 * v + lane;
    if (f >= ngroups) continue;
    float4 a = W > 1 ? add4(acc0[v], acc1[v]) : acc0[v];
    float4 r = make_float4(alpha * a.x, alpha * a.y, alpha * a.z, alpha * a.w);
    float* o = out + 4 * f;
    if (4 * f + 4 <= n) {
      if (beta != 0.f) {
        const float4 old = load4_nt(o);
        r.x = r.x + beta * old.x;
        r.y = r.y + beta * old.y;
        r.z = r.z + beta * old.z;
        r.w = r.w + beta * old.w;
      }
      store4_nt(o, r);
    } else {
      const int rem = (int)(n - 4 * f);
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        if (k < rem) {
          float rk = comp(r, k);
          if (beta != 0.f) rk = rk + beta * o[k];
          o[k] = rk;
        }
      }
    }
  }
}

template <int SCHEME, int BITS>
__global__ __launch_bounds__(kThreads) void k_error_feedback(
    int64_t n, int dsh, int s, int L, const float* __restrict__ g,
    float* __restrict__ e, const uint8_t* __restrict__ codes,
    const float* __restrict__ meta, int64_t code_bytes, DenseCfg dc) {
  const int64_t ngroups = (n + 3) >> 2;
  const int64_t f0 = (int64_t)blockIdx.x * kGroupsPerBlock + threadIdx.x;
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    const int64_t f = f0 + (int64_t)kThreads * v;
    if (f >= ngroups) continue;
    const int64_t i = 4 * f;
    const bool full = i + 4 <= n;
    const float4 x = dequant4<SCHEME, BITS>(
        load_group<BITS>(codes, f, full, code_bytes, dc), meta, i >> dsh, s, L);
    const float4 gv = full ? load4_nt(g + i) : load4(g, i, n);
    const float4 ev = full ? load4_nt(e + i) : load4(e, i, n);
    float4 r;
    r.x = (gv.x + ev.x) - x.x;
    r.y = (gv.y + ev.y) - x.y;
    r.z = (gv.z + ev.z) - x.z;
    r.w = (gv.w + ev.w) - x.w;
    if (full) store4_nt(e + i, r);
    else store4(e, i, n, r);
  }
}

// Per-layer scale (TernGrad, "Gradient Quantization" glossary, ternary
// paragraph): the uniform scheme with layer l = elements [off[l], off[l+1])
// as one bucket.  Same tiles and accumulation order as k_deq_acc; the step
// of each element is that of its layer, M / s, divided once per (payload,
// layer) of the tile into LDS (per element for a tile met by more than
// kMaxStarts layers).
static_assert(kThreads == 256, "find_tile_layers expects blocks of 256 threads");

template <int BITS, int NB>
__global__ __launch_bounds__(kThreads) void k_layer_deq(
    int64_t n, int nl, const int64_t* __restrict__ off, int s, int W,
    PayloadPtrs pp, float alpha, float beta, float* __restrict__ out,
    int64_t code_bytes, DenseCfg dc) {
  __shared__ TileLayers T;
  __shared__ float dtab[kMaxPayloads][kMaxStarts + 1];
  const int64_t ngroups = (n + 3) >> 2;
  const int64_t tile = (int64_t)blockIdx.x * kGroupsPerBlock;
  const int64_t f0 = tile + threadIdx.x;
  const int64_t t0 = 4 * tile;
  const int64_t t1 = t0 + 4 * (int64_t)kGroupsPerBlock < n ? t0 + 4 * (int64_t)kGroupsPerBlock : n;
  int64_t o[kOffPerThread];
  prefetch_offsets(o, off, nl);
  // the first batch of code loads goes out before the layer search
  uint32_t cw[NB][kV];
  auto load_batch = [&](int p0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int p = p0 + j;
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        const int64_t f = f0 + (int64_t)kThreads * v;
        cw[j][v] = (p < W && f < ngroups)
                       ? load_group<BITS>(pp.codes[p < W ? p : 0], f,
                                          4 * f + 4 <= n, code_bytes, dc)
                       : 0u;
      }
    }
  };
  load_batch(0);
  int lf, ns;
  find_tile_layers(T, o, off, nl, t0, t1, lf, ns);
  // a tile inside one layer (ns = 0, block-uniform) reads each payload's
  // step itself, without the LDS table and its barrier
  if (ns != 0) {
    const int nent = ns > 0 ? ns + 1 : 0;
    for (int t = threadIdx.x; t < W * nent; t += kThreads)
      dtab[t / nent][t % nent] = pp.meta[t / nent][lf + t % nent] / (float)s;
    __syncthreads();
  }
  float dl[NB];  // ns = 0: the batch's steps
  auto batch_steps = [&](int p0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int p = p0 + j;
      dl[j] = (ns == 0 && p < W) ? pp.meta[p][lf] / (float)s : 0.f;
    }
  };
  batch_steps(0);

  // layer of each element (ns != 0): its LDS column, or (ns < 0) the layer
  int li[kV][4];
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    const int64_t i = 4 * (f0 + (int64_t)kThreads * v);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      li[v][k] = 0;
      if (ns != 0) {
        const int l = elem_layer(T, lf, ns, off, nl, i + k < n ? i + k : n - 1);
        li[v][k] = ns > 0 ? l - lf : l;
      }
    }
  }
  float4 acc0[kV], acc1[kV];
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    acc0[v] = make_float4(0.f, 0.f, 0.f, 0.f);
    acc1[v] = acc0[v];
  }
  for (int p0 = 0; p0 < W; p0 += NB) {
    if (p0 > 0) {
      load_batch(p0);
      batch_steps(p0);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int p = p0 + j;
      if (p >= W) break;
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        const int64_t f = f0 + (int64_t)kThreads * v;
        if (f >= ngroups) continue;
        float x[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float delta = ns == 0 ? dl[j]
                              : (ns > 0 ? dtab[p][li[v][k]]
                                        : pp.meta[p][li[v][k]] / (float)s);
          x[k] = (float)code_value<UNIFORM, BITS>(cw[j][v], k, s) * delta;
        }
        const float4 xv = make_float4(x[0], x[1], x[2], x[3]);
        if (p == 0) acc0[v] = xv;
        else if (p == 1) acc1[v] = xv;
        else if (p & 1) acc1[v] = add4(acc1[v], xv);
        else acc0[v] = add4(acc0[v], xv);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    const int64_t f = f0 + (int64_t)kThreads * v;
    if (f >= ngroups) continue;
    float4 a = W > 1 ? add4(acc0[v], acc1[v]) : acc0[v];
    float4 r = make_float4(alpha * a.x, alpha * a.y, alpha * a.z, alpha * a.w);
    float* o = out + 4 * f;
    if (4 * f + 4 <= n) {
      if (beta != 0.f) {
        const float4 old = load4_nt(o);
        r.x = r.x + beta * old.x;
        r.y = r.y + beta * old.y;
        r.z = r.z + beta * old.z;
        r.w = r.w + beta * old.w;
      }
      store4_nt(o, r);
    } else {
      const int rem = (int)(n - 4 * f);
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        if (k < rem) {
          float rk = comp(r, k);
          if (beta != 0.f) rk = rk + beta * o[k];
          o[k] = rk;
        }
      }
    }
  }
}

int64_t blocks_for(int64_t n) {
  const int64_t ngroups = (n + 3) >> 2;
  return (ngroups + kGroupsPerBlock - 1) / kGroupsPerBlock;
}

DenseCfg dense_cfg(const LaunchDesc& L) {
  DenseCfg dc{L.W, (uint32_t)L.A, L.A4, {0.0, 0.0, 0.f, 0.f}};
  if (L.dense) {
    dc.r.rA4 = 1.0 / (double)L.A4;
    dc.r.hA4 = 0.5 * dc.r.rA4;
    dc.r.rA = 1.0f / (float)L.A;
    dc.r.hA = 0.5f * dc.r.rA;
  }
  return dc;
}

// log2 of the bucket size (a power of two)
int dshift(const LaunchDesc& L) { return __builtin_ctz((unsigned)L.d); }

template <int SCHEME, int BITS>
int deq_wide(const LaunchDesc& L, int64_t n, int W, const PayloadPtrs& pp,
             float alpha, float beta, float* out, int64_t code_bytes,
             hipStream_t st) {
  const int64_t ngroups = (n + 3) >> 2;
  const dim3 grid((uint32_t)((ngroups + kWideBlockGroups - 1) / kWideBlockGroups)),
      block(kThreads);
  // payloads whose codes together exceed the 256 MiB last-level cache are
  // streamed past it (measured: INT8, W = 8, n = 256M 537 -> 512 us; on
  // cache-resident payloads the hint costs up to 25 %)
  const bool nt = (double)W * (double)code_bytes > 256.0 * 1024 * 1024;
#define GQ_WIDE(NB, NT)                                                          \
  hipLaunchKernelGGL((k_deq_acc_wide<SCHEME, BITS, NB, NT>), grid, block, 0, st, \
                     n, dshift(L), L.s, L.L, W, pp, alpha, beta, out,            \
                     code_bytes)
  if (W == 1) { if (nt) GQ_WIDE(1, true); else GQ_WIDE(1, false); }
  else if (W == 2) { if (nt) GQ_WIDE(2, true); else GQ_WIDE(2, false); }
  else if (W <= 4) { if (nt) GQ_WIDE(4, true); else GQ_WIDE(4, false); }
  else { if (nt) GQ_WIDE(8, true); else GQ_WIDE(8, false); }
#undef GQ_WIDE
  return (int)hipGetLastError();
}

template <int SCHEME, int BITS>
int deq_one(const LaunchDesc& L, int64_t n, int W, const PayloadPtrs& pp,
            float alpha, float beta, float* out, int64_t code_bytes,
            hipStream_t st) {
  if constexpr ((BITS == 4 || BITS == 8) && (SCHEME == UNIFORM || SCHEME == ORQ))
    return deq_wide<SCHEME, BITS>(L, n, W, pp, alpha, beta, out, code_bytes, st);
  const dim3 grid((uint32_t)blocks_for(n)), block(kThreads);
  const DenseCfg dc = dense_cfg(L);
  if (W == 1)
    hipLaunchKernelGGL((k_deq_acc<SCHEME, BITS, 1>), grid, block, 0, st, n,
                       dshift(L), L.s, L.L, W, pp, alpha, beta, out, code_bytes, dc);
  else if (W == 2)
    hipLaunchKernelGGL((k_deq_acc<SCHEME, BITS, 2>), grid, block, 0, st, n,
                       dshift(L), L.s, L.L, W, pp, alpha, beta, out, code_bytes, dc);
  else
    hipLaunchKernelGGL((k_deq_acc<SCHEME, BITS, 4>), grid, block, 0, st, n,
                       dshift(L), L.s, L.L, W, pp, alpha, beta, out, code_bytes, dc);
  return (int)hipGetLastError();
}

template <int SCHEME, int BITS>
int ef_one(const LaunchDesc& L, int64_t n, const float* g, float* e,
           const uint8_t* codes, const float* meta, int64_t code_bytes,
           hipStream_t st) {
  hipLaunchKernelGGL((k_error_feedback<SCHEME, BITS>),
                     dim3((uint32_t)blocks_for(n)), dim3(kThreads), 0, st, n,
                     dshift(L), L.s, L.L, g, e, codes, meta, code_bytes,
                     dense_cfg(L));
  return (int)hipGetLastError();
}

// Calls F<SCHEME, BITS>(args...) for the descriptor's (scheme, bits);
// BITS = 0 for dense packing.
#define GQ_DISPATCH(FN, ...)                                        \
  if (L.dense) {                                                    \
    if (L.scheme == UNIFORM) return FN<UNIFORM, 0>(__VA_ARGS__);    \
    if (L.scheme == ORQ) return FN<ORQ, 0>(__VA_ARGS__);            \
    return (int)hipErrorInvalidValue;                               \
  }                                                                 \
  switch (L.scheme) {                                               \
    case UNIFORM:                                                   \
      switch (L.bits) {                                             \
        case 2: return FN<UNIFORM, 2>(__VA_ARGS__);                 \
        case 3: return FN<UNIFORM, 3>(__VA_ARGS__);                 \
        case 4: return FN<UNIFORM, 4>(__VA_ARGS__);                 \
        case 8: return FN<UNIFORM, 8>(__VA_ARGS__);                 \
        default: return (int)hipErrorInvalidValue;                  \
      }                                                             \
    case BIN_SIGN:                                                  \
    case BIN_OPT:                                                   \
      return FN<BIN_SIGN, 1>(__VA_ARGS__);                          \
    case ORQ:                                                       \
      switch (L.bits) {                                             \
        case 1: return FN<ORQ, 1>(__VA_ARGS__);                     \
        case 2: return FN<ORQ, 2>(__VA_ARGS__);                     \
        case 3: return FN<ORQ, 3>(__VA_ARGS__);                     \
        case 4: return FN<ORQ, 4>(__VA_ARGS__);                     \
        default: return (int)hipErrorInvalidValue;                  \
      }                                                             \
    default:                                                        \
      return (int)hipErrorInvalidValue;                             \
  }

template <int BITS>
int layer_deq_one(const LaunchDesc& L, int64_t n, int nl, const int64_t* off,
                  int W, const PayloadPtrs& pp, float alpha, float beta,
                  float* out, int64_t code_bytes, hipStream_t st) {
  const dim3 grid((uint32_t)blocks_for(n)), block(kThreads);
  const DenseCfg dc = dense_cfg(L);
  if (W == 1)
    hipLaunchKernelGGL((k_layer_deq<BITS, 1>), grid, block, 0, st, n, nl, off,
                       L.s, W, pp, alpha, beta, out, code_bytes, dc);
  else if (W == 2)
    hipLaunchKernelGGL((k_layer_deq<BITS, 2>), grid, block, 0, st, n, nl, off,
                       L.s, W, pp, alpha, beta, out, code_bytes, dc);
  else
    hipLaunchKernelGGL((k_layer_deq<BITS, 4>), grid, block, 0, st, n, nl, off,
                       L.s, W, pp, alpha, beta, out, code_bytes, dc);
  return (int)hipGetLastError();
}

}  // namespace

int launch_deq_acc(const LaunchDesc& L, int64_t n, int W, const PayloadPtrs& pp,
                   float alpha, float beta, float* out, int64_t code_bytes,
                   hipStream_t st) {
  GQ_DISPATCH(deq_one, L, n, W, pp, alpha, beta, out, code_bytes, st)
}

int launch_error_feedback(const LaunchDesc& L, int64_t n, const float* g,
                          float* e, const uint8_t* codes, const float* meta,
                          int64_t code_bytes, hipStream_t st) {
  GQ_DISPATCH(ef_one, L, n, g, e, codes, meta, code_bytes, st)
}

}  // namespace gq

namespace gq {

int launch_layer_deq(const LaunchDesc& L, int64_t n, int nl,
                     const int64_t* off, int W, const PayloadPtrs& pp,
                     float alpha, float beta, float* out, int64_t code_bytes,
                     hipStream_t st) {
  if (L.scheme != UNIFORM) return (int)hipErrorInvalidValue;
  if (L.dense) return layer_deq_one<0>(L, n, nl, off, W, pp, alpha, beta, out, code_bytes, st);
  switch (L.bits) {
    case 2: return layer_deq_one<2>(L, n, nl, off, W, pp, alpha, beta, out, code_bytes, st);
    case 3: return layer_deq_one<3>(L, n, nl, off, W, pp, alpha, beta, out, code_bytes, st);
    case 4: return layer_deq_one<4>(L, n, nl, off, W, pp, alpha, beta, out, code_bytes, st);
    case 8: return layer_deq_one<8>(L, n, nl, off, W, pp, alpha, beta, out, code_bytes, st);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace gq
