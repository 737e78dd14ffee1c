// deq.hip — decompress side: unpack, dequantize and accumulate W payloads
// into an fp32 average ("gradient quantization for communication" glossary,
// §How Gradient Quantization Works: dequantize, then aggregate), and the
// standalone residual update of error feedback ("Gradient Quantization"
// glossary, error-feedback paragraph).
//
// Output-stationary: each thread owns 16 consecutive output elements (all in
// one bucket, since d >= 64 is a multiple of 16).  Per payload it reads the
// 2*BITS code bytes of those elements with one load, the bucket's meta row,
// decodes 16 codes and adds them into two fp32 accumulators (even and odd
// payloads), so a sum of W terms is at most ceil(W/2)+1 additions deep.
#include "common.hpp"

namespace gq {
namespace {

constexpr int kElems = 16;   // elements per thread
constexpr int kThreads = 256;

// Code bytes of the thread's 16 elements: 2*BITS bytes at 2*BITS*t.  The
// full path uses one aligned load; the last thread of a partial payload
// reads byte by byte up to code_bytes.
template <int BITS>
__device__ __forceinline__ void load_chunk(const uint8_t* __restrict__ c,
                                           int64_t t, bool full,
                                           int64_t code_bytes, uint32_t w[4]) {
  const int64_t off = (int64_t)2 * BITS * t;
  w[0] = w[1] = w[2] = w[3] = 0u;
  if (full) {
    if constexpr (BITS == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(c + off);
      w[0] = v.x;
      w[1] = v.y;
      w[2] = v.z;
      w[3] = v.w;
    } else if constexpr (BITS == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(c + off);
      w[0] = v.x;
      w[1] = v.y;
    } else if constexpr (BITS == 2) {
      w[0] = *reinterpret_cast<const uint32_t*>(c + off);
    } else if constexpr (BITS == 1) {
      w[0] = *reinterpret_cast<const uint16_t*>(c + off);
    } else {  // 3 bits: 6 bytes, 2-byte aligned
      const uint16_t* h = reinterpret_cast<const uint16_t*>(c + off);
      w[0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
      w[1] = (uint32_t)h[2];
    }
  } else {
    for (int b = 0; b < 2 * BITS; ++b)
      if (off + b < code_bytes) w[b >> 2] |= (uint32_t)c[off + b] << (8 * (b & 3));
  }
}

template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t w[4], int k) {
  const int o = BITS * k;
  if constexpr (BITS == 3) {
    const uint64_t x = (uint64_t)w[0] | ((uint64_t)w[1] << 32);
    return (uint32_t)(x >> o) & 7u;
  } else {
    return (w[o >> 5] >> (o & 31)) & ((1u << BITS) - 1u);
  }
}

// Dequantized value of the 16 codes of one payload.
template <int SCHEME, int BITS>
__device__ __forceinline__ void dequant16(const uint32_t w[4],
                                          const float* __restrict__ meta,
                                          int64_t bucket, int s, int L,
                                          float x[kElems]) {
  if constexpr (SCHEME == UNIFORM) {
    const float delta = meta[bucket] / (float)s;
#pragma unroll
    for (int k = 0; k < kElems; ++k) {
      const uint32_t u = code_at<BITS>(w, k);
      const uint32_t m = 1u << (BITS - 1);
      const int ci = (int)((u ^ m) - m);  // sign-extend
      x[k] = (float)ci * delta;
    }
  } else if constexpr (SCHEME == BIN_SIGN || SCHEME == BIN_OPT) {
    const float a = meta[2 * bucket + 0], b = meta[2 * bucket + 1];
#pragma unroll
    for (int k = 0; k < kElems; ++k) x[k] = code_at<BITS>(w, k) ? b : a;
  } else {
    // codes past the level table (never written by the quantizer) are
    // clamped so that no read leaves the bucket's meta row
    const float* lv = meta + bucket * L;
    const uint32_t top = (uint32_t)(L - 1);
#pragma unroll
    for (int k = 0; k < kElems; ++k) {
      const uint32_t c = code_at<BITS>(w, k);
      x[k] = lv[c < top ? c : top];
    }
  }
}

template <int SCHEME, int BITS>
__global__ __launch_bounds__(kThreads) void k_deq_acc(
    int64_t n, int d, int s, int L, int W, PayloadPtrs pp, float alpha,
    float beta, float* __restrict__ out, int64_t code_bytes) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t i0 = t * kElems;
  if (i0 >= n) return;
  const bool full = i0 + kElems <= n;
  const int64_t bucket = i0 / d;

  float acc0[kElems], acc1[kElems];
  {
    uint32_t w[4];
    load_chunk<BITS>(pp.codes[0], t, full, code_bytes, w);
    dequant16<SCHEME, BITS>(w, pp.meta[0], bucket, s, L, acc0);
  }
  if (W > 1) {
    uint32_t w[4];
    load_chunk<BITS>(pp.codes[1], t, full, code_bytes, w);
    dequant16<SCHEME, BITS>(w, pp.meta[1], bucket, s, L, acc1);
  }
  for (int p = 2; p < W; ++p) {
    uint32_t w[4];
    float x[kElems];
    load_chunk<BITS>(pp.codes[p], t, full, code_bytes, w);
    dequant16<SCHEME, BITS>(w, pp.meta[p], bucket, s, L, x);
    if (p & 1) {
#pragma unroll
      for (int k = 0; k < kElems; ++k) acc1[k] = acc1[k] + x[k];
    } else {
#pragma unroll
      for (int k = 0; k < kElems; ++k) acc0[k] = acc0[k] + x[k];
    }
  }
  if (W > 1) {
#pragma unroll
    for (int k = 0; k < kElems; ++k) acc0[k] = acc0[k] + acc1[k];
  }

  float* o = out + i0;
  if (full) {
#pragma unroll
    for (int q = 0; q < kElems / 4; ++q) {
      float4 r;
      r.x = alpha * acc0[4 * q + 0];
      r.y = alpha * acc0[4 * q + 1];
      r.z = alpha * acc0[4 * q + 2];
      r.w = alpha * acc0[4 * q + 3];
      if (beta != 0.f) {
        const float4 old = reinterpret_cast<const float4*>(o)[q];
        r.x = r.x + beta * old.x;
        r.y = r.y + beta * old.y;
        r.z = r.z + beta * old.z;
        r.w = r.w + beta * old.w;
      }
      reinterpret_cast<float4*>(o)[q] = r;
    }
  } else {
    for (int k = 0; k < kElems; ++k) {
      if (i0 + k < n) {
        float r = alpha * acc0[k];
        if (beta != 0.f) r = r + beta * o[k];
        o[k] = r;
      }
    }
  }
}

template <int SCHEME, int BITS>
__global__ __launch_bounds__(kThreads) void k_error_feedback(
    int64_t n, int d, int s, int L, const float* __restrict__ g,
    float* __restrict__ e, const uint8_t* __restrict__ codes,
    const float* __restrict__ meta, int64_t code_bytes) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t i0 = t * kElems;
  if (i0 >= n) return;
  const bool full = i0 + kElems <= n;
  uint32_t w[4];
  float x[kElems];
  load_chunk<BITS>(codes, t, full, code_bytes, w);
  dequant16<SCHEME, BITS>(w, meta, i0 / d, s, L, x);
  if (full) {
#pragma unroll
    for (int q = 0; q < kElems / 4; ++q) {
      const float4 gv = reinterpret_cast<const float4*>(g + i0)[q];
      const float4 ev = reinterpret_cast<const float4*>(e + i0)[q];
      float4 r;
      r.x = (gv.x + ev.x) - x[4 * q + 0];
      r.y = (gv.y + ev.y) - x[4 * q + 1];
      r.z = (gv.z + ev.z) - x[4 * q + 2];
      r.w = (gv.w + ev.w) - x[4 * q + 3];
      reinterpret_cast<float4*>(e + i0)[q] = r;
    }
  } else {
    for (int k = 0; k < kElems; ++k)
      if (i0 + k < n) e[i0 + k] = (g[i0 + k] + e[i0 + k]) - x[k];
  }
}

template <int SCHEME, int BITS>
int deq_one(const LaunchDesc& L, int64_t n, int W, const PayloadPtrs& pp,
            float alpha, float beta, float* out, int64_t code_bytes,
            hipStream_t st) {
  const int64_t threads = (n + kElems - 1) / kElems;
  const int64_t blocks = (threads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((k_deq_acc<SCHEME, BITS>), dim3((uint32_t)blocks),
                     dim3(kThreads), 0, st, n, L.d, L.s, L.L, W, pp, alpha,
                     beta, out, code_bytes);
  return (int)hipGetLastError();
}

template <int SCHEME, int BITS>
int ef_one(const LaunchDesc& L, int64_t n, const float* g, float* e,
           const uint8_t* codes, const float* meta, int64_t code_bytes,
           hipStream_t st) {
  const int64_t threads = (n + kElems - 1) / kElems;
  const int64_t blocks = (threads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((k_error_feedback<SCHEME, BITS>), dim3((uint32_t)blocks),
                     dim3(kThreads), 0, st, n, L.d, L.s, L.L, g, e, codes, meta,
                     code_bytes);
  return (int)hipGetLastError();
}

// Calls F<SCHEME, BITS>(args...) for the descriptor's (scheme, bits).
#define GQ_DISPATCH(FN, ...)                                        \
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
