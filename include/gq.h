/*
 * gq.h — C ABI of libgq: bucketed stochastic gradient quantization with
 * error feedback, for AMD Instinct MI355X (gfx950).
 *
 * The operations are the compress / decompress / aggregate steps of
 * data-parallel gradient exchange ("gradient quantization for
 * communication" glossary, §How Gradient Quantization Works: quantize before
 * transmission, dequantize on receipt, then average) together with the
 * error-feedback loop ("Gradient Quantization" glossary, error-feedback
 * paragraph: keep the quantization residual and add it to the next
 * gradient).  One GPU; no collectives.
 *
 * Layout shared by every call
 *   - A gradient is a flat fp32 array of n >= 1 elements.  Bucket j holds
 *     elements [j*d, min(n, (j+1)*d)); the last bucket may be partial and its
 *     statistics use only its real elements ("Optimal Gradient Quantization
 *     Condition" review, §Proposed method: fixed-size buckets, d = 512).
 *   - Codes form one LSB-first bitstream: element i owns stream bits
 *     [b*i, b*i + b), stream bit t is bit (t mod 8) of byte t/8, code bit 0
 *     first.  Bytes past the last element's bits are written as zero.
 *   - With GQ_FLAG_DENSE the stream holds fields of W bits instead: eight
 *     consecutive codes form one base-A integer (A = 2s+1 symbols for
 *     GQ_UNIFORM, digit c + s; A = L for GQ_ORQ, digit = level index), the
 *     first code least significant, absent codes of a partial group 0, and
 *     field g occupies stream bits [W*g, W*g + W), W = ceil(log2 A^8)
 *     (ternary 13 bits per 8 codes, nine levels 26): the compression the
 *     paper review quotes for ORQ-3 / ORQ-9 (20.2 / 10.1 x, the entropy
 *     limit 32/log2 A) is reached to within 2.5 %.
 *   - meta is fp32 [nb][k]:  k = 1 (GQ_UNIFORM: the bucket's max-abs M),
 *     2 (GQ_BIN_*: lower level a, upper level b), L (GQ_ORQ: ascending levels).
 *
 * Conventions
 *   - All pointers to arrays are DEVICE pointers (except the two pointer
 *     arrays of gq_dequantize_accumulate, which live in host memory and hold
 *     device pointers).  Every device array must be 16-byte aligned.
 *   - The caller owns every buffer; libgq allocates no device memory and
 *     keeps no state between calls, so calls on different streams may run
 *     concurrently as long as their buffers do not overlap.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; nothing synchronizes the device.
 *   - Argument errors are detected on the host before any launch and
 *     returned; a failed launch returns GQ_ELAUNCH.  A GPU dispatch holds
 *     fewer than 2^32 work-items, which bounds n per call for the kernels
 *     with a thread per few elements: about 2^35 for the quantizers and
 *     the dequantizer at d >= 512 (2^34 at d = 64), 2^26 * d for GQ_TOPK
 *     (a wave per bucket); beyond that a launch fails, the call returns GQ_ELAUNCH
 *     and its outputs are unspecified.  The Elias calls stride and take
 *     any n.
 *   - Inputs must be finite; NaN/Inf inputs give unspecified outputs but
 *     never out-of-bounds accesses.
 *   - Outputs are a pure function of (inputs, desc, seed, step): they do not
 *     depend on launch configuration or on other calls.
 */
#ifndef GQ_H
#define GQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Schemes.
 * GQ_UNIFORM  max-abs scaled uniform levels, s per sign, random rounding:
 *             QSGD (s = 4: 4-bit), ternary / TernGrad (s = 1: 2-bit),
 *             INT8 (s = 127).  ("Gradient Quantization" glossary: core
 *             mechanism, Stochastic Quantization bullet, QSGD and ternary
 *             paragraphs.)
 * GQ_BIN_SIGN two levels split at zero, each the mean of its side; 1-bit
 *             (the sign path: ternary/binary paragraph, SignSGD).
 * GQ_BIN_OPT  two levels minimising the bucket's squared error (BinGrad-b:
 *             "Optimal Gradient Quantization Condition" review, §Proposed
 *             method); deterministic, 1-bit.
 * GQ_ORQ      L levels picked greedily to minimise the summed random-
 *             rounding variance sum (b-x)(x-a), random rounding between
 *             adjacent levels (ORQ, same section); optional clip.  With
 *             L = 2 the levels are the bucket's minimum and maximum: the
 *             unbiased wide-range two-level quantizer the review contrasts
 *             with BinGrad-b (BinGrad-pb, as read here).
 * GQ_TOPK     Top-K sparsification combined with quantization ("gradient
 *             quantization for communication" glossary, §Quantization
 *             Schemes): per bucket only the K = desc.levels elements of
 *             largest |p| are sent (all of a bucket with fewer; equal
 *             magnitudes: the lower index first), each rounded on the
 *             bucket's uniform grid of s levels per sign exactly as
 *             GQ_UNIFORM rounds it (same scale M = max |p|, same Philox
 *             word); the others decode as 0 and stay in the residual.
 *             d <= 512, 1 <= K <= d, flags: GQ_FLAG_NEAREST only.  Codes:
 *             bucket j owns R = ceil(K (log2 d + b) / 32) 32-bit words at
 *             byte 4 R j (b = the GQ_UNIFORM code width); slot t, the t-th
 *             kept element in increasing index, holds its index within the
 *             bucket (log2 d bits) then its code (b bits, two's complement)
 *             at bits [t w, t w + w) of the record, w = log2 d + b, LSB
 *             first; unused slots and pad bits are 0.  meta: the bucket's
 *             max-abs.  gq_code_bits reports w.  gq_select_levels and
 *             gq_error_feedback return GQ_EUNSUPPORTED (gq_quantize writes
 *             the residual). */
typedef enum {
  GQ_UNIFORM = 0,
  GQ_BIN_SIGN = 1,
  GQ_BIN_OPT = 2,
  GQ_ORQ = 3,
  GQ_TOPK = 4
} gq_scheme;

/* GQ_FLAG_CLIP (GQ_ORQ only): clip every value of a bucket to
 * +-clip_sigma * RMS(bucket) before selecting levels and rounding (same
 * section: clipping).
 * GQ_FLAG_DENSE: dense packing of the codes (see the layout above): for
 * GQ_UNIFORM with s <= 7 and for GQ_ORQ with d >= 512 (GQ_EUNSUPPORTED
 * otherwise).  For the two-level schemes and ORQ with L a power of two the
 * dense layout is the fixed-width layout, and the flag changes nothing.
 * Every call that reads or writes a payload must be given the same flag.
 * GQ_FLAG_NEAREST (GQ_UNIFORM and GQ_ORQ): deterministic rounding to the
 * nearest level instead of random rounding ("Gradient Quantization"
 * glossary, Deterministic Quantization bullet): with q the value's
 * fractional position between its two adjacent levels, it rounds up iff
 * q > 1/2 (a value exactly halfway takes the lower level, i.e. the smaller
 * magnitude for GQ_UNIFORM).  This is the random rule with u = 1/2 for every
 * element; seed and step are ignored.  The two-level schemes are already
 * deterministic and return GQ_EUNSUPPORTED for it.  Payloads are read the
 * same way with or without the flag.
 * GQ_FLAG_BISECT (GQ_ORQ with d <= 512): the levels by recursive bisection,
 * the other reading of the review's greedy selection (same section; its
 * 3 / 5 / 9 levels are 2^k + 1): rounds in which every interval between
 * adjacent levels receives its own best level at once; a round that would
 * pass L levels inserts its largest gains first (equal gains: the smaller
 * value).  Without the flag one level is inserted per step, the one with
 * the largest gain over all intervals.  GQ_EUNSUPPORTED for other schemes
 * and for d > 512. */
enum { GQ_FLAG_CLIP = 1, GQ_FLAG_DENSE = 2, GQ_FLAG_NEAREST = 4, GQ_FLAG_BISECT = 8 };

typedef struct {
  int32_t scheme;     /* gq_scheme                                          */
  int32_t bucket;     /* d: power of two, 64 <= d <= 32768                  */
  int32_t s;          /* GQ_UNIFORM: levels per sign, 1..127                 */
  int32_t levels;     /* GQ_ORQ: L total levels incl. min and max, 2..16     */
  int32_t flags;      /* GQ_FLAG_* bits (others must be 0)                  */
  float clip_sigma;   /* with GQ_FLAG_CLIP: > 0                             */
} gq_desc;

enum {
  GQ_OK = 0,
  GQ_EINVAL = -1,       /* null/misaligned pointer, bad size or descriptor  */
  GQ_EUNSUPPORTED = -2, /* well-formed but unsupported (scheme, s, L, flag) */
  GQ_ELAUNCH = -3,      /* a kernel launch failed (hipGetLastError)         */
  GQ_ETOOMANY = -4      /* W > GQ_MAX_PAYLOADS                               */
};

#define GQ_MAX_PAYLOADS 16

/* Bits per code: GQ_UNIFORM ceil(log2(2s+1)) rounded up to 2, 3, 4 or 8
 * (two's complement); GQ_BIN_* 1 (1 = upper level); GQ_ORQ ceil(log2 L)
 * (unsigned level index).  With GQ_FLAG_DENSE (where it changes the
 * layout): the width W of one 8-code field.  Host-only; never touches the
 * GPU. */
int gq_code_bits(const gq_desc* desc, int32_t* bits);

/* Payload sizes for n elements: code_bytes = ceil(n*bits/8) (dense:
 * ceil(ceil(n/8)*W/8)); meta_floats = ceil(n/d) * k.  A codes buffer that
 * gq_quantize writes must hold code_bytes rounded up to a multiple of 16
 * (it stores whole 32-bit words; the bytes past code_bytes are written as
 * 0).  Either output pointer may be NULL.  Host-only. */
int gq_payload_size(const gq_desc* desc, int64_t n, int64_t* code_bytes,
                    int64_t* meta_floats);

/* Per-bucket levels of p = g (+ e when e != NULL) into meta, exactly as
 * gq_quantize would compute them; nothing else is written. */
int gq_select_levels(const gq_desc* desc, int64_t n, const float* g,
                     const float* e, float* meta, void* stream);

/* Quantize n elements: p = g (+ e), levels per bucket, random rounding
 * (round up iff u < q, u from Philox4x32-10 with key = seed and counter =
 * (i/4, step); element i uses word i mod 4, u = (word >> 8) * 2^-24; with
 * GQ_FLAG_NEAREST u = 1/2), pack.
 * With e != NULL, e is read and then overwritten in place with the residual
 * p - dequant(code) (unclipped p).  codes: code_bytes rounded up to a
 * multiple of 16 bytes.  e must not
 * overlap g, codes or meta. */
int gq_quantize(const gq_desc* desc, int64_t n, const float* g, float* e,
                uint64_t seed, uint32_t step, uint8_t* codes, float* meta,
                void* stream);

/* Standalone residual update: e <- fl(fl(g + e) - dequant(codes, meta));
 * bitwise equal to the residual gq_quantize writes for the same payload. */
int gq_error_feedback(const gq_desc* desc, int64_t n, const float* g, float* e,
                      const uint8_t* codes, const float* meta, void* stream);

/* Aggregate W payloads (1 <= W <= GQ_MAX_PAYLOADS), each quantized with the
 * same desc over the same n:  out <- beta*out + alpha * sum_w dequant_w.
 * codes[w] / meta[w] are device pointers held in HOST arrays of length W.
 * beta == 0 means out is write-only (never read).  Accumulation is fp32;
 * W = 1, alpha = 1, beta = 0 reproduces dequant exactly.  out must not
 * overlap any payload. */
int gq_dequantize_accumulate(const gq_desc* desc, int64_t n, int32_t W,
                             const uint8_t* const* codes,
                             const float* const* meta, float alpha, float beta,
                             float* out, void* stream);

/* Per-layer scale ("Gradient Quantization" glossary, ternary paragraph:
 * TernGrad keeps one scaling factor per layer).  The gradient is the
 * concatenation of nl >= 1 layers: layer l = elements
 * [layer_offsets[l], layer_offsets[l+1]) of the flat array, with
 * layer_offsets a DEVICE array of nl + 1 int64 values, 8-byte aligned,
 * layer_offsets[0] = 0, layer_offsets[nl] = n, non-decreasing (empty layers
 * allowed).  Each layer is one bucket of GQ_UNIFORM whatever its size:
 * meta holds nl floats, meta[l] = max |p| over layer l (0 if empty), and
 * every code is rounded on its own layer's grid exactly as in gq_quantize.
 * Codes, Philox counter (the flat element index) and dense layout are
 * those of gq_quantize for the flat array.  desc->scheme must be
 * GQ_UNIFORM (GQ_EUNSUPPORTED otherwise; GQ_FLAG_DENSE and GQ_FLAG_NEAREST
 * apply, desc->bucket is not used but must be valid).  The offsets are not
 * read on the host: other contents give unspecified outputs but never
 * out-of-bounds accesses.  Two passes over g (and e): the layer maxima
 * first (meta is zeroed by the call), then rounding, packing and the
 * residual.  meta, codes and e must not overlap layer_offsets or g. */
int gq_quantize_layers(const gq_desc* desc, int64_t n, int32_t nl,
                       const int64_t* layer_offsets, const float* g, float* e,
                       uint64_t seed, uint32_t step, uint8_t* codes,
                       float* meta, void* stream);

/* gq_dequantize_accumulate for payloads written by gq_quantize_layers with
 * the same desc, n and layer layout (meta[w] holds nl floats). */
int gq_dequantize_accumulate_layers(const gq_desc* desc, int64_t n, int32_t nl,
                                    const int64_t* layer_offsets, int32_t W,
                                    const uint8_t* const* codes,
                                    const float* const* meta, float alpha,
                                    float beta, float* out, void* stream);

/* Layer-wise bit allocation ("Gradient Quantization" glossary, layer-wise
 * quantization paragraph: wider codes for layers with larger gradient
 * variance; the page gives no rule).  For the per-layer scale path: each of
 * the nl <= 1024 layers (layer_offsets as in gq_quantize_layers) gets a
 * width b in {2, 3, 4, 8}, with s = 2^(b-1) - 1 levels per sign.  All start
 * at 2; the upgrades 2->3, 3->4, 4->8 of every layer are ranked by the
 * reduction of the layer's bound n_l * M_l^2 / (4 s^2) on its rounding
 * variance per added bit, M_l^2 * (1/s_b^2 - 1/s_b'^2) / (4 (b' - b)) in
 * fp64 (M_l = scales[l], e.g. the meta gq_quantize_layers writes), equal
 * values by layer, then width, and taken in that order up to the first
 * that would pass budget_bits total code bits (budget_bits >= 2 n;
 * upgrades that reduce nothing end the list; empty layers keep 2).
 * Outputs (DEVICE): widths[nl] int32, segments[nl + 1] int64 byte offsets
 * of each layer's code segment in a payload of the allocation (its n_l
 * codes at its width, padded to 16 bytes; segments[nl] = payload bytes).
 * GQ_EUNSUPPORTED for nl > 1024.  One block on the stream; offsets are not
 * read on the host (other contents: unspecified outputs, in-bounds
 * accesses). */
int gq_allocate_layer_bits(int64_t n, int32_t nl, const int64_t* layer_offsets,
                           const float* scales, int64_t budget_bits,
                           int32_t* widths, int64_t* segments, void* stream);

/* Capacity a payload of any allocation needs: n + 16 nl bytes (every code at
 * 8 bits plus every segment's padding).  GQ_EINVAL for n or nl out of range
 * or a null bytes. */
int gq_alloc_payload_bytes(int64_t n, int32_t nl, int64_t* bytes);

/* Quantize with a layer-wise bit allocation (same glossary paragraph): the
 * per-layer scale path of gq_quantize_layers with layer l coded at
 * widths[l] bits, s = 2^(b-1) - 1, the uniform scheme.  Inputs as in
 * gq_quantize_layers (g, e, layer_offsets, seed, step; flags: 0 or
 * GQ_FLAG_NEAREST) plus widths[nl] int32 and segments[nl + 1] int64 (DEVICE,
 * as gq_allocate_layer_bits writes them: widths in {2, 3, 4, 8}, segments
 * the 16-byte-padded byte offsets).  Outputs (DEVICE): meta[nl] fp32 = each
 * layer's max-abs of p = g (+ e); payload bytes [segments[l],
 * segments[l+1]) = layer l's n_l codes as an LSB-first bit stream (code k at
 * bits [k b, k b + b), two's complement), zero past the last code; e <- p -
 * x_hat when e is given.  A layer's codes are exactly those gq_quantize_layers
 * gives with s = 2^(b-1) - 1 (same scale, Philox word per flat index and
 * rounding).  payload_bytes >= gq_alloc_payload_bytes(n, nl) (GQ_EINVAL
 * otherwise); bytes past segments[nl] are not written.  Alignment: g, e,
 * payload, meta 16 bytes; layer_offsets and segments 8; widths 4.  No buffer
 * written may overlap another buffer of the call.  Device tables are not
 * read on the host: a width outside {2, 3, 4, 8} writes zero codes for that
 * layer and leaves its residual unspecified (the identity e = p - x_hat is
 * kept only for layers of a valid width), and other contents (segments off
 * 16-byte boundaries, offsets that disagree with the segments) give
 * unspecified outputs but only in-bounds stores.  Two launches on the
 * stream (max-abs, codes). */
int gq_quantize_layers_alloc(int64_t n, int32_t nl, const int64_t* layer_offsets,
                             const float* g, float* e, const int32_t* widths,
                             const int64_t* segments, uint64_t seed,
                             uint32_t step, int32_t flags, uint8_t* payload,
                             int64_t payload_bytes, float* meta, void* stream);

/* out <- beta * out + alpha * sum_w x_hat_w over W <= GQ_MAX_PAYLOADS
 * payloads of gq_quantize_layers_alloc (one layer layout; each payload has
 * its own meta[w], widths[w] and segments[w], DEVICE, alignments as
 * above).  Summation order as in gq_dequantize_accumulate.  GQ_ETOOMANY for
 * W > GQ_MAX_PAYLOADS; GQ_EINVAL for null or misaligned pointers, a
 * non-finite alpha or beta, or out overlapping layer_offsets, a table, a
 * scale array or the start of a payload.  The payloads are read within
 * [0, segments[w][nl]) when widths and segments are those the allocation
 * wrote; other contents are the caller's error. */
int gq_dequantize_accumulate_layers_alloc(
    int64_t n, int32_t nl, const int64_t* layer_offsets, int32_t W,
    const uint8_t* const* payloads, const float* const* meta,
    const int32_t* const* widths, const int64_t* const* segments, float alpha,
    float beta, float* out, void* stream);

/* Elias gamma coding of GQ_UNIFORM codes, the lossless integer coding QSGD
 * applies after quantizing ("Gradient Quantization" glossary, QSGD
 * paragraph).  Code c (in element order) is written as the Elias gamma code
 * of m = |c| + 1 (floor(log2 m) zero bits, then the floor(log2 m) + 1 binary
 * digits of m, most significant first) followed, when c != 0, by one sign
 * bit (1 = negative): 0 takes 1 bit, +-1 and +-2 take 4, +-3 .. +-6 take 6.
 * Stream bit t is bit t mod 32 of 32-bit word t / 32.  Each bucket's record
 * starts on a word; pad bits are 0.  offsets: nb + 1 uint64 word offsets,
 * offsets[j] = first word of bucket j's record, offsets[0] = 0,
 * offsets[nb] = words used; a receiver needs them with the words.
 * desc: GQ_UNIFORM without GQ_FLAG_DENSE (GQ_EUNSUPPORTED otherwise;
 * GQ_FLAG_NEAREST does not change the codes' layout). */

/* Words the stream needs at most: every code with |c| = s.  Host-only. */
int gq_elias_max_words(const gq_desc* desc, int64_t n, int64_t* max_words);

/* Encode the n codes of a gq_quantize payload (codes: code_bytes rounded
 * up to 16, fixed-width layout) into words (gq_elias_max_words words) and offsets
 * (nb + 1).  Codes outside [-s, s] (never written by gq_quantize) are
 * clamped to that range.  Three launches; offsets doubles as the scan's
 * workspace, so no other memory is used.  codes, offsets and words must not
 * overlap. */
int gq_elias_encode(const gq_desc* desc, int64_t n, const uint8_t* codes,
                    uint64_t* offsets, uint32_t* words, void* stream);

/* Decode an Elias stream back into the fixed-width codes gq_quantize wrote
 * (bit-identical for a stream from gq_elias_encode), ready for
 * gq_dequantize_accumulate.  n_words >= 1: the readable length of words
 * (reads stay below it; offsets are clamped to it).  Writes
 * ceil(code_bytes / 4) 32-bit words of codes (capacity: code_bytes rounded
 * up to 16).  A corrupt stream gives unspecified codes but no out-of-bounds
 * access. */
int gq_elias_decode(const gq_desc* desc, int64_t n, const uint64_t* offsets,
                    const uint32_t* words, int64_t n_words, uint8_t* codes,
                    void* stream);

/* Static description of a status code. */
const char* gq_strerror(int status);

/* Library version, (major << 16) | minor. */
int gq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GQ_H */
