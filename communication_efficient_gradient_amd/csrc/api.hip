// api.hip — the C ABI declared in include/gq.h: argument validation on the
// host, then dispatch to the kernel launchers.  No allocation, no global
// state, no device synchronization.
#include "gq.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "common.hpp"

namespace {

constexpr int64_t kMaxN = int64_t(1) << 38;  // beyond any single HBM stack

int ceil_log2(int v) {
  int b = 0;
  while ((1 << b) < v) ++b;
  return b;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// Validates a descriptor and fills the launch parameters.
int check_desc(const gq_desc* d, gq::LaunchDesc* L) {
  if (d == nullptr) return GQ_EINVAL;
  const int b = d->bucket;
  if (b < 64 || b > 32768 || (b & (b - 1)) != 0) return GQ_EINVAL;
  if (d->flags & ~(GQ_FLAG_CLIP | GQ_FLAG_DENSE | GQ_FLAG_NEAREST | GQ_FLAG_BISECT))
    return GQ_EINVAL;
  L->scheme = d->scheme;
  L->d = b;
  L->s = d->s;
  L->L = d->levels;
  L->flags = d->flags;
  L->clip_sigma = d->clip_sigma;
  switch (d->scheme) {
    case GQ_UNIFORM: {
      if (d->s < 1 || d->s > 127) return GQ_EUNSUPPORTED;
      const int w = ceil_log2(2 * d->s + 1);
      L->bits = w <= 4 ? w : 8;
      L->k = 1;
      break;
    }
    case GQ_BIN_SIGN:
    case GQ_BIN_OPT:
      L->bits = 1;
      L->k = 2;
      break;
    case GQ_ORQ:
      if (d->levels < 2 || d->levels > 16) return GQ_EUNSUPPORTED;
      L->bits = ceil_log2(d->levels);
      L->k = d->levels;
      break;
    case GQ_TOPK: {
      // K = levels kept per bucket; values on the uniform grid of s levels
      if (d->s < 1 || d->s > 127 || b > 512) return GQ_EUNSUPPORTED;
      if (d->levels < 1 || d->levels > b) return GQ_EINVAL;
      const int w = ceil_log2(2 * d->s + 1);
      L->bits = w <= 4 ? w : 8;
      L->k = 1;
      if (d->flags & ~GQ_FLAG_NEAREST) return GQ_EUNSUPPORTED;
      break;
    }
    default:
      return GQ_EUNSUPPORTED;
  }
  if (d->flags & GQ_FLAG_CLIP) {
    if (d->scheme != GQ_ORQ) return GQ_EUNSUPPORTED;
    if (!(d->clip_sigma > 0.f) || !std::isfinite(d->clip_sigma)) return GQ_EINVAL;
  }
  if ((d->flags & GQ_FLAG_NEAREST) && d->scheme != GQ_UNIFORM && d->scheme != GQ_ORQ &&
      d->scheme != GQ_TOPK)
    return GQ_EUNSUPPORTED;
  if ((d->flags & GQ_FLAG_BISECT) && (d->scheme != GQ_ORQ || b > 512))
    return GQ_EUNSUPPORTED;
  L->dense = 0;
  L->A = L->W = 0;
  L->A4 = 0;
  if (d->flags & GQ_FLAG_DENSE) {
    const int A = d->scheme == GQ_UNIFORM ? 2 * d->s + 1
                                          : (d->scheme == GQ_ORQ ? d->levels : 2);
    if (A > 16) return GQ_EUNSUPPORTED;
    if ((A & (A - 1)) != 0) {  // not a power of two: a different layout
      if (d->scheme == GQ_ORQ && b < 512) return GQ_EUNSUPPORTED;
      uint64_t p = 1;
      for (int i = 0; i < 8; ++i) p *= (uint64_t)A;
      int w = 0;
      while (((uint64_t)1 << w) < p) ++w;
      L->dense = 1;
      L->A = A;
      L->W = w;
      L->A4 = (uint32_t)(A * A * A * A);
      L->bits = w;  // reported by gq_code_bits as the 8-code field width
    }
  }
  return GQ_OK;
}

int64_t code_bytes_of(const gq::LaunchDesc& L, int64_t n) {
  if (L.scheme == GQ_TOPK)
    return ((n + L.d - 1) / L.d) * 4 * (int64_t)gq::topk_record_words(L.d, L.bits, L.L);
  if (L.dense) return (((n + 7) / 8) * L.W + 7) / 8;
  return (n * L.bits + 7) / 8;
}
int64_t meta_floats_of(const gq::LaunchDesc& L, int64_t n) {
  return ((n + L.d - 1) / L.d) * L.k;
}

int launch_status(int hip_rc) { return hip_rc == 0 ? GQ_OK : GQ_ELAUNCH; }

// ORQ with two levels and no clipping keeps the bucket's minimum and
// maximum: a reduction, so it runs in the streaming quantizer.
bool is_sort_scheme(const gq::LaunchDesc& L) {
  if (L.scheme == GQ_ORQ && L.L == 2 && !(L.flags & GQ_FLAG_CLIP)) return false;
  return L.scheme == GQ_BIN_OPT || L.scheme == GQ_ORQ;
}

}  // namespace

extern "C" {

int gq_version(void) { return (1 << 16) | 0; }

const char* gq_strerror(int status) {
  switch (status) {
    case GQ_OK:
      return "success";
    case GQ_EINVAL:
      return "invalid argument (null or misaligned pointer, bad size, bad descriptor, overlapping buffers)";
    case GQ_EUNSUPPORTED:
      return "unsupported scheme parameters";
    case GQ_ELAUNCH:
      return "kernel launch failed";
    case GQ_ETOOMANY:
      return "too many payloads (W > GQ_MAX_PAYLOADS)";
    default:
      return "unknown status";
  }
}

int gq_code_bits(const gq_desc* desc, int32_t* bits) {
  gq::LaunchDesc L;
  const int rc = check_desc(desc, &L);
  if (rc) return rc;
  if (bits == nullptr) return GQ_EINVAL;
  // Top-K: one slot = bucket index bits + code bits
  *bits = L.scheme == GQ_TOPK ? ceil_log2(L.d) + L.bits : L.bits;
  return GQ_OK;
}

int gq_payload_size(const gq_desc* desc, int64_t n, int64_t* code_bytes,
                    int64_t* meta_floats) {
  gq::LaunchDesc L;
  const int rc = check_desc(desc, &L);
  if (rc) return rc;
  if (n < 1 || n > kMaxN) return GQ_EINVAL;
  if (code_bytes) *code_bytes = code_bytes_of(L, n);
  if (meta_floats) *meta_floats = meta_floats_of(L, n);
  return GQ_OK;
}

int gq_select_levels(const gq_desc* desc, int64_t n, const float* g,
                     const float* e, float* meta, void* stream) {
  gq::LaunchDesc L;
  int rc = check_desc(desc, &L);
  if (rc) return rc;
  if (L.scheme == GQ_TOPK) return GQ_EUNSUPPORTED;
  if (n < 1 || n > kMaxN || !g || !meta) return GQ_EINVAL;
  if (!aligned16(g) || !aligned16(meta) || (e && !aligned16(e))) return GQ_EINVAL;
  if (overlap(meta, 4 * meta_floats_of(L, n), g, 4 * n) ||
      (e && overlap(meta, 4 * meta_floats_of(L, n), e, 4 * n)))
    return GQ_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* ew = const_cast<float*>(e);  // read-only when codes == nullptr
  if (is_sort_scheme(L))
    return launch_status(gq::launch_sort_quant(L, n, g, ew, 0, 0, nullptr, meta,
                                               0, st));
  return launch_status(gq::launch_stream_quant(L, n, g, ew, 0, 0, nullptr, meta,
                                               0, st));
}

int gq_quantize(const gq_desc* desc, int64_t n, const float* g, float* e,
                uint64_t seed, uint32_t step, uint8_t* codes, float* meta,
                void* stream) {
  gq::LaunchDesc L;
  int rc = check_desc(desc, &L);
  if (rc) return rc;
  if (n < 1 || n > kMaxN || !g || !codes || !meta) return GQ_EINVAL;
  if (!aligned16(g) || !aligned16(codes) || !aligned16(meta) || (e && !aligned16(e)))
    return GQ_EINVAL;
  const int64_t cb = code_bytes_of(L, n);
  const int64_t cap = (cb + 15) / 16 * 16;
  const int64_t mb = 4 * meta_floats_of(L, n);
  if (e && (overlap(e, 4 * n, g, 4 * n) || overlap(e, 4 * n, codes, cap) ||
            overlap(e, 4 * n, meta, mb)))
    return GQ_EINVAL;
  if (overlap(codes, cap, g, 4 * n) || overlap(meta, mb, g, 4 * n) ||
      overlap(codes, cap, meta, mb))
    return GQ_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (L.scheme == GQ_TOPK)
    return launch_status(gq::launch_topk_quant(L, n, g, e, seed, step, codes, meta, st));
  if (is_sort_scheme(L))
    return launch_status(
        gq::launch_sort_quant(L, n, g, e, seed, step, codes, meta, cb, st));
  return launch_status(
      gq::launch_stream_quant(L, n, g, e, seed, step, codes, meta, cb, st));
}

int gq_error_feedback(const gq_desc* desc, int64_t n, const float* g, float* e,
                      const uint8_t* codes, const float* meta, void* stream) {
  gq::LaunchDesc L;
  int rc = check_desc(desc, &L);
  if (rc) return rc;
  if (L.scheme == GQ_TOPK) return GQ_EUNSUPPORTED;
  if (n < 1 || n > kMaxN || !g || !e || !codes || !meta) return GQ_EINVAL;
  if (!aligned16(g) || !aligned16(e) || !aligned16(codes) || !aligned16(meta))
    return GQ_EINVAL;
  const int64_t cb = code_bytes_of(L, n);
  if (overlap(e, 4 * n, g, 4 * n) || overlap(e, 4 * n, codes, cb) ||
      overlap(e, 4 * n, meta, 4 * meta_floats_of(L, n)))
    return GQ_EINVAL;
  return launch_status(gq::launch_error_feedback(
      L, n, g, e, codes, meta, cb, static_cast<hipStream_t>(stream)));
}

int gq_dequantize_accumulate(const gq_desc* desc, int64_t n, int32_t W,
                             const uint8_t* const* codes,
                             const float* const* meta, float alpha, float beta,
                             float* out, void* stream) {
  gq::LaunchDesc L;
  int rc = check_desc(desc, &L);
  if (rc) return rc;
  if (W > GQ_MAX_PAYLOADS) return GQ_ETOOMANY;
  if (n < 1 || n > kMaxN || W < 1 || !codes || !meta || !out) return GQ_EINVAL;
  if (!aligned16(out) || !std::isfinite(alpha) || !std::isfinite(beta))
    return GQ_EINVAL;
  const int64_t cb = code_bytes_of(L, n);
  const int64_t mb = 4 * meta_floats_of(L, n);
  gq::PayloadPtrs pp{};
  for (int w = 0; w < W; ++w) {
    if (!codes[w] || !meta[w] || !aligned16(codes[w]) || !aligned16(meta[w]))
      return GQ_EINVAL;
    if (overlap(out, 4 * n, codes[w], cb) || overlap(out, 4 * n, meta[w], mb))
      return GQ_EINVAL;
    pp.codes[w] = codes[w];
    pp.meta[w] = meta[w];
  }
  if (L.scheme == GQ_TOPK)
    return launch_status(gq::launch_topk_deq(L, n, W, pp, alpha, beta, out,
                                             static_cast<hipStream_t>(stream)));
  return launch_status(gq::launch_deq_acc(L, n, W, pp, alpha, beta, out, cb,
                                          static_cast<hipStream_t>(stream)));
}

int gq_quantize_layers(const gq_desc* desc, int64_t n, int32_t nl,
                       const int64_t* layer_offsets, const float* g, float* e,
                       uint64_t seed, uint32_t step, uint8_t* codes,
                       float* meta, void* stream) {
  gq::LaunchDesc L;
  int rc = check_desc(desc, &L);
  if (rc) return rc;
  if (L.scheme != GQ_UNIFORM) return GQ_EUNSUPPORTED;
  if (n < 1 || n > kMaxN || nl < 1 || !layer_offsets || !g || !codes || !meta)
    return GQ_EINVAL;
  if (!aligned16(g) || !aligned16(codes) || !aligned16(meta) ||
      (e && !aligned16(e)) || reinterpret_cast<uintptr_t>(layer_offsets) % 8)
    return GQ_EINVAL;
  const int64_t cb = code_bytes_of(L, n);
  const int64_t cap = (cb + 15) / 16 * 16;
  const int64_t mb = 4 * (int64_t)nl, ob = 8 * ((int64_t)nl + 1);
  if (e && (overlap(e, 4 * n, g, 4 * n) || overlap(e, 4 * n, codes, cap) ||
            overlap(e, 4 * n, meta, mb) || overlap(e, 4 * n, layer_offsets, ob)))
    return GQ_EINVAL;
  if (overlap(codes, cap, g, 4 * n) || overlap(meta, mb, g, 4 * n) ||
      overlap(codes, cap, meta, mb) || overlap(codes, cap, layer_offsets, ob) ||
      overlap(meta, mb, layer_offsets, ob))
    return GQ_EINVAL;
  return launch_status(gq::launch_layer_quant(L, n, nl, layer_offsets, g, e,
                                              seed, step, codes, meta, cb,
                                              static_cast<hipStream_t>(stream)));
}

int gq_allocate_layer_bits(int64_t n, int32_t nl, const int64_t* layer_offsets,
                           const float* scales, int64_t budget_bits,
                           int32_t* widths, int64_t* segments, void* stream) {
  if (n < 1 || n > kMaxN || nl < 1 || !layer_offsets || !scales || !widths ||
      !segments || budget_bits < 2 * n)
    return GQ_EINVAL;
  if (nl > 1024) return GQ_EUNSUPPORTED;
  if (!aligned16(scales) || !aligned16(widths) || !aligned16(segments) ||
      reinterpret_cast<uintptr_t>(layer_offsets) % 8)
    return GQ_EINVAL;
  const int64_t ob = 8 * ((int64_t)nl + 1), sb = 4 * (int64_t)nl;
  if (overlap(widths, sb, layer_offsets, ob) || overlap(widths, sb, scales, sb) ||
      overlap(segments, ob, layer_offsets, ob) || overlap(segments, ob, scales, sb) ||
      overlap(widths, sb, segments, ob))
    return GQ_EINVAL;
  return launch_status(gq::launch_layer_alloc(nl, layer_offsets, scales,
                                              budget_bits, widths, segments,
                                              static_cast<hipStream_t>(stream)));
}

// Room for the payload of any allocation: every code at 8 bits plus the
// padding of every segment.
static int64_t alloc_capacity(int64_t n, int32_t nl) { return n + 16 * (int64_t)nl; }

int gq_alloc_payload_bytes(int64_t n, int32_t nl, int64_t* bytes) {
  if (n < 1 || n > kMaxN || nl < 1 || !bytes) return GQ_EINVAL;
  *bytes = alloc_capacity(n, nl);
  return GQ_OK;
}

int gq_quantize_layers_alloc(int64_t n, int32_t nl, const int64_t* layer_offsets,
                             const float* g, float* e, const int32_t* widths,
                             const int64_t* segments, uint64_t seed,
                             uint32_t step, int32_t flags, uint8_t* payload,
                             int64_t payload_bytes, float* meta, void* stream) {
  if (n < 1 || n > kMaxN || nl < 1 || !layer_offsets || !g || !widths ||
      !segments || !payload || !meta || (flags & ~GQ_FLAG_NEAREST))
    return GQ_EINVAL;
  if (payload_bytes < alloc_capacity(n, nl)) return GQ_EINVAL;
  if (!aligned16(g) || !aligned16(payload) || !aligned16(meta) ||
      (e && !aligned16(e)) || reinterpret_cast<uintptr_t>(layer_offsets) % 8 ||
      reinterpret_cast<uintptr_t>(widths) % 4 ||
      reinterpret_cast<uintptr_t>(segments) % 8)
    return GQ_EINVAL;
  const int64_t mb = 4 * (int64_t)nl, ob = 8 * ((int64_t)nl + 1);
  const int64_t pb = payload_bytes;
  const void* in[4] = {layer_offsets, widths, segments, g};
  const int64_t in_b[4] = {ob, mb, ob, 4 * n};
  for (int k = 0; k < 4; ++k) {
    if (overlap(payload, pb, in[k], in_b[k]) || overlap(meta, mb, in[k], in_b[k]) ||
        (e && overlap(e, 4 * n, in[k], in_b[k])))
      return GQ_EINVAL;
  }
  if (overlap(payload, pb, meta, mb) || (e && (overlap(e, 4 * n, payload, pb) ||
                                              overlap(e, 4 * n, meta, mb))))
    return GQ_EINVAL;
  return launch_status(gq::launch_alloc_quant(
      n, nl, layer_offsets, g, e, widths, segments, seed, step,
      (flags & GQ_FLAG_NEAREST) ? 1 : 0, payload, payload_bytes, meta,
      static_cast<hipStream_t>(stream)));
}

int gq_dequantize_accumulate_layers_alloc(
    int64_t n, int32_t nl, const int64_t* layer_offsets, int32_t W,
    const uint8_t* const* payloads, const float* const* meta,
    const int32_t* const* widths, const int64_t* const* segments, float alpha,
    float beta, float* out, void* stream) {
  if (W > GQ_MAX_PAYLOADS) return GQ_ETOOMANY;
  if (n < 1 || n > kMaxN || nl < 1 || W < 1 || !layer_offsets || !payloads ||
      !meta || !widths || !segments || !out)
    return GQ_EINVAL;
  if (!aligned16(out) || reinterpret_cast<uintptr_t>(layer_offsets) % 8 ||
      !std::isfinite(alpha) || !std::isfinite(beta))
    return GQ_EINVAL;
  const int64_t mb = 4 * (int64_t)nl, ob = 8 * ((int64_t)nl + 1);
  if (overlap(out, 4 * n, layer_offsets, ob)) return GQ_EINVAL;
  for (int w = 0; w < W; ++w) {
    if (!payloads[w] || !meta[w] || !widths[w] || !segments[w] ||
        !aligned16(payloads[w]) || !aligned16(meta[w]) ||
        reinterpret_cast<uintptr_t>(widths[w]) % 4 ||
        reinterpret_cast<uintptr_t>(segments[w]) % 8)
      return GQ_EINVAL;
    // a payload's size lives on the device (segments[nl]); its first
    // 16 bytes, the tables and the scales must lie outside out
    if (overlap(out, 4 * n, payloads[w], 16) || overlap(out, 4 * n, meta[w], mb) ||
        overlap(out, 4 * n, widths[w], mb) || overlap(out, 4 * n, segments[w], ob))
      return GQ_EINVAL;
  }
  return launch_status(gq::launch_alloc_deq(n, nl, layer_offsets, W, payloads,
                                            meta, widths, segments, alpha,
                                            beta, out,
                                            static_cast<hipStream_t>(stream)));
}

int gq_dequantize_accumulate_layers(const gq_desc* desc, int64_t n, int32_t nl,
                                    const int64_t* layer_offsets, int32_t W,
                                    const uint8_t* const* codes,
                                    const float* const* meta, float alpha,
                                    float beta, float* out, void* stream) {
  gq::LaunchDesc L;
  int rc = check_desc(desc, &L);
  if (rc) return rc;
  if (L.scheme != GQ_UNIFORM) return GQ_EUNSUPPORTED;
  if (W > GQ_MAX_PAYLOADS) return GQ_ETOOMANY;
  if (n < 1 || n > kMaxN || nl < 1 || W < 1 || !layer_offsets || !codes ||
      !meta || !out)
    return GQ_EINVAL;
  if (!aligned16(out) || reinterpret_cast<uintptr_t>(layer_offsets) % 8 ||
      !std::isfinite(alpha) || !std::isfinite(beta))
    return GQ_EINVAL;
  const int64_t cb = code_bytes_of(L, n);
  const int64_t mb = 4 * (int64_t)nl, ob = 8 * ((int64_t)nl + 1);
  if (overlap(out, 4 * n, layer_offsets, ob)) return GQ_EINVAL;
  gq::PayloadPtrs pp{};
  for (int w = 0; w < W; ++w) {
    if (!codes[w] || !meta[w] || !aligned16(codes[w]) || !aligned16(meta[w]))
      return GQ_EINVAL;
    if (overlap(out, 4 * n, codes[w], cb) || overlap(out, 4 * n, meta[w], mb))
      return GQ_EINVAL;
    pp.codes[w] = codes[w];
    pp.meta[w] = meta[w];
  }
  return launch_status(gq::launch_layer_deq(L, n, nl, layer_offsets, W, pp,
                                            alpha, beta, out, cb,
                                            static_cast<hipStream_t>(stream)));
}

// Elias gamma coding: GQ_UNIFORM payloads in the fixed-width layout only.
static int check_elias(const gq_desc* desc, int64_t n, gq::LaunchDesc* L) {
  int rc = check_desc(desc, L);
  if (rc) return rc;
  if (L->scheme != GQ_UNIFORM || L->dense) return GQ_EUNSUPPORTED;
  if (n < 1 || n > kMaxN) return GQ_EINVAL;
  return GQ_OK;
}

int gq_elias_max_words(const gq_desc* desc, int64_t n, int64_t* max_words) {
  gq::LaunchDesc L;
  int rc = check_elias(desc, n, &L);
  if (rc) return rc;
  if (!max_words) return GQ_EINVAL;
  *max_words = gq::elias_max_words(L, n);
  return GQ_OK;
}

int gq_elias_encode(const gq_desc* desc, int64_t n, const uint8_t* codes,
                    uint64_t* offsets, uint32_t* words, void* stream) {
  gq::LaunchDesc L;
  int rc = check_elias(desc, n, &L);
  if (rc) return rc;
  if (!codes || !offsets || !words) return GQ_EINVAL;
  if (!aligned16(codes) || !aligned16(offsets) || !aligned16(words)) return GQ_EINVAL;
  const int64_t cap = (code_bytes_of(L, n) + 15) / 16 * 16;
  const int64_t ob = 8 * ((n + L.d - 1) / L.d + 1);
  const int64_t wb = 4 * gq::elias_max_words(L, n);
  if (overlap(codes, cap, offsets, ob) || overlap(codes, cap, words, wb) ||
      overlap(offsets, ob, words, wb))
    return GQ_EINVAL;
  return launch_status(gq::launch_elias_encode(L, n, codes, offsets, words,
                                               static_cast<hipStream_t>(stream)));
}

int gq_elias_decode(const gq_desc* desc, int64_t n, const uint64_t* offsets,
                    const uint32_t* words, int64_t n_words, uint8_t* codes,
                    void* stream) {
  gq::LaunchDesc L;
  int rc = check_elias(desc, n, &L);
  if (rc) return rc;
  if (!codes || !offsets || !words || n_words < 1) return GQ_EINVAL;
  if (!aligned16(codes) || !aligned16(offsets) || !aligned16(words)) return GQ_EINVAL;
  const int64_t cap = (code_bytes_of(L, n) + 15) / 16 * 16;
  const int64_t ob = 8 * ((n + L.d - 1) / L.d + 1);
  if (overlap(codes, cap, offsets, ob) || overlap(codes, cap, words, 4 * n_words))
    return GQ_EINVAL;
  return launch_status(gq::launch_elias_decode(L, n, offsets, words, n_words,
                                               codes,
                                               static_cast<hipStream_t>(stream)));
}

}  // extern "C"
