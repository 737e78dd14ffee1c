"""CPU oracle for bucketed stochastic gradient quantization (numpy front end).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library itself never does.
It wraps ``libgqref.so`` (plain scalar C, ``gqref.c``) with numpy arrays and
shares no code with the HIP library.

Parity status of each routine (what pins it is in ``tests/test_oracle_*``):
    philox                rocRAND's philox4x32_10 run on the host; bit
                          frequency and chi-square statistics
    quantize (uniform)    0.7 example, unbiasedness over seeds, variance
                          closed form and QSGD bound, code range,
                          deterministic special cases, EF identity
    quantize (bin_sign)   numpy side means, SSE(opt) <= SSE(sign)
    quantize (bin_opt)    brute force over all 2^d partitions / all splits
    quantize (orq)        brute-force best insertion per greedy step, global
                          optimum for L=3, grid search, variance chain
    pack / unpack         numpy.packbits (1 bit), int8 bytes (8 bit)
    dense pack / unpack   Python big-integer base-A arithmetic, field widths
                          from exact integer powers, round trips
    dequantize_accumulate exact rational sums (fractions) on small inputs
    elias encode / decode textbook gamma codewords (golden file), a bit-string
                          parser written in the test, lengths from the
                          code-length formula, round trips
    allocate_layer_bits   brute force over every allocation of small
                          layouts (exact rational bounds), monotone widths,
                          budget extremes
    *_layers_alloc        values on each layer's grid next to p, exact
                          residual, segment sizes and padding, exact
                          rational aggregation, one width = per-layer path
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

UNIFORM, BIN_SIGN, BIN_OPT, ORQ = 0, 1, 2, 3
FLAG_CLIP = 1
FLAG_DENSE = 2
FLAG_NEAREST = 4
FLAG_BISECT = 8

_lib = None


def lib():
    global _lib
    if _lib is None:
        # GQREF_LIBRARY: another build of gqref.c (the sanitizer test loads
        # an AddressSanitizer / UBSan build through it)
        path = os.environ.get("GQREF_LIBRARY")
        if path is None:
            if _build.needs_build():
                _build.build()
            path = _build.LIB
        L = C.CDLL(path)
        i64, u64, u32, i32 = C.c_int64, C.c_uint64, C.c_uint32, C.c_int
        fp, cfp, u8p = C.c_void_p, C.c_void_p, C.c_void_p
        L.gqref_philox.argtypes = [u64, u64, u32, C.POINTER(C.c_uint32)]
        L.gqref_philox.restype = None
        L.gqref_philox_blocks.argtypes = [u64, u64, i64, u32, C.c_void_p]
        L.gqref_philox_blocks.restype = None
        L.gqref_bits.argtypes = [i32, i32, i32]
        L.gqref_meta_per_bucket.argtypes = [i32, i32]
        L.gqref_quantize.argtypes = [i32, i32, i32, i32, i32, C.c_float, i64,
                                     i64, cfp, fp, u64, u32, u8p, fp, u8p]
        L.gqref_select_levels.argtypes = [i32, i32, i32, i32, i32, C.c_float,
                                          i64, i64, cfp, cfp, fp, u8p]
        L.gqref_dequantize.argtypes = [i32, i32, i32, i32, i32, i64, u8p, cfp,
                                       fp]
        L.gqref_error_feedback.argtypes = [i32, i32, i32, i32, i32, i64, cfp,
                                           fp, u8p, cfp]
        L.gqref_dequantize_accumulate.argtypes = [
            i32, i32, i32, i32, i32, i64, i32, C.POINTER(C.c_void_p),
            C.POINTER(C.c_void_p), C.c_float, C.c_float, fp]
        L.gqref_quantize_layers.argtypes = [i32, i32, i64, i32, C.c_void_p,
                                            cfp, fp, u64, u32, u8p, fp]
        L.gqref_dequantize_accumulate_layers.argtypes = [
            i32, i32, i64, i32, C.c_void_p, i32, C.POINTER(C.c_void_p),
            C.POINTER(C.c_void_p), C.c_float, C.c_float, fp]
        L.gqref_topk_record_words.argtypes = [i32, i32, i32]
        L.gqref_quantize_topk.argtypes = [i32, i32, i32, i32, i64, cfp, fp,
                                          u64, u32, u8p, fp]
        L.gqref_dequantize_accumulate_topk.argtypes = [
            i32, i32, i32, i32, i64, i32, C.POINTER(C.c_void_p),
            C.POINTER(C.c_void_p), C.c_float, C.c_float, fp]
        L.gqref_elias_max_words.argtypes = [i32, i32, i64]
        L.gqref_elias_max_words.restype = i64
        L.gqref_elias_encode.argtypes = [i32, i32, i64, u8p, C.c_void_p,
                                         C.c_void_p]
        L.gqref_elias_decode.argtypes = [i32, i32, i64, C.c_void_p, C.c_void_p,
                                         u8p]
        L.gqref_dense_width.argtypes = [i32]
        L.gqref_pack_dense.argtypes = [i32, i64, C.c_void_p, u8p]
        L.gqref_pack_dense.restype = None
        L.gqref_unpack_dense.argtypes = [i32, i64, u8p, C.c_void_p]
        L.gqref_unpack_dense.restype = None
        L.gqref_pack.argtypes = [i32, i64, C.c_void_p, u8p]
        L.gqref_pack.restype = None
        L.gqref_unpack.argtypes = [i32, i64, u8p, C.c_void_p]
        L.gqref_unpack.restype = None
        L.gqref_set_threads.argtypes = [i32]
        L.gqref_set_threads.restype = None
        _lib = L
    return _lib


@dataclass(frozen=True)
class Desc:
    """Scheme parameters (bucket size d, s levels per sign, L ORQ levels)."""
    scheme: int = UNIFORM
    d: int = 512
    s: int = 4
    L: int = 5
    flags: int = 0
    clip_sigma: float = 3.0

    @property
    def bits(self) -> int:
        return lib().gqref_bits(self.scheme, self.s, self.L)

    @property
    def k(self) -> int:
        return lib().gqref_meta_per_bucket(self.scheme, self.L)

    @property
    def dense(self) -> bool:
        return bool(self.flags & FLAG_DENSE)

    @property
    def alphabet(self) -> int:
        """Number of distinct codes: 2s+1, L or 2."""
        return 2 * self.s + 1 if self.scheme == UNIFORM else (
            self.L if self.scheme == ORQ else 2)

    @property
    def field_bits(self) -> int:
        """Dense packing: bits of one 8-code field."""
        return dense_width(self.alphabet)

    def nb(self, n: int) -> int:
        return (n + self.d - 1) // self.d

    def code_bytes(self, n: int) -> int:
        if self.dense:
            return (((n + 7) // 8) * self.field_bits + 7) // 8
        return (n * self.bits + 7) // 8


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def set_threads(t: int) -> None:
    lib().gqref_set_threads(int(t))


def threads() -> int:
    return lib().gqref_get_threads()


def philox(seed: int, ctr: int, step: int) -> np.ndarray:
    out = (C.c_uint32 * 4)()
    lib().gqref_philox(seed, ctr, step, out)
    return np.array(out[:], dtype=np.uint32)


def philox_blocks(seed: int, ctr0: int, nblocks: int, step: int) -> np.ndarray:
    out = np.empty((nblocks, 4), dtype=np.uint32)
    lib().gqref_philox_blocks(seed, ctr0, nblocks, step, out.ctypes.data)
    return out


def quantize(desc: Desc, g, e=None, seed: int = 0, step: int = 0, i0: int = 0):
    """Returns (codes u8, meta f32[nb, k], e_new or None, tie u8[nb])."""
    g = _f32(g)
    n = g.size
    e_new = None if e is None else _f32(e).copy()
    codes = np.zeros(desc.code_bytes(n), dtype=np.uint8)
    meta = np.zeros((desc.nb(n), desc.k), dtype=np.float32)
    tie = np.zeros(desc.nb(n), dtype=np.uint8)
    rc = lib().gqref_quantize(desc.scheme, desc.d, desc.s, desc.L, desc.flags,
                              desc.clip_sigma, i0, n, _ptr(g), _ptr(e_new),
                              seed, step, _ptr(codes), _ptr(meta), _ptr(tie))
    if rc:
        raise ValueError("oracle quantize: invalid arguments")
    return codes, meta, e_new, tie


def select_levels(desc: Desc, g, e=None, i0: int = 0):
    g = _f32(g)
    e = None if e is None else _f32(e)
    n = g.size
    meta = np.zeros((desc.nb(n), desc.k), dtype=np.float32)
    tie = np.zeros(desc.nb(n), dtype=np.uint8)
    rc = lib().gqref_select_levels(desc.scheme, desc.d, desc.s, desc.L,
                                   desc.flags, desc.clip_sigma, i0, n, _ptr(g),
                                   _ptr(e), _ptr(meta), _ptr(tie))
    if rc:
        raise ValueError("oracle select_levels: invalid arguments")
    return meta, tie


def dequantize(desc: Desc, n: int, codes, meta):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    meta = _f32(meta)
    out = np.empty(n, dtype=np.float32)
    rc = lib().gqref_dequantize(desc.scheme, desc.d, desc.s, desc.L,
                                desc.flags, n, _ptr(codes), _ptr(meta),
                                _ptr(out))
    if rc:
        raise ValueError("oracle dequantize: invalid arguments")
    return out


def error_feedback(desc: Desc, g, e, codes, meta):
    g = _f32(g)
    e = _f32(e).copy()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    meta = _f32(meta)
    rc = lib().gqref_error_feedback(desc.scheme, desc.d, desc.s, desc.L,
                                    desc.flags, g.size, _ptr(g), _ptr(e),
                                    _ptr(codes), _ptr(meta))
    if rc:
        raise ValueError("oracle error_feedback: invalid arguments")
    return e


def dequantize_accumulate(desc: Desc, n: int, codes_list, meta_list,
                          alpha: float = 1.0, beta: float = 0.0, out=None):
    W = len(codes_list)
    cl = [np.ascontiguousarray(c, dtype=np.uint8) for c in codes_list]
    ml = [_f32(m) for m in meta_list]
    out = np.zeros(n, dtype=np.float32) if out is None else _f32(out).copy()
    cp = (C.c_void_p * W)(*[c.ctypes.data for c in cl])
    mp = (C.c_void_p * W)(*[m.ctypes.data for m in ml])
    rc = lib().gqref_dequantize_accumulate(desc.scheme, desc.d, desc.s, desc.L,
                                           desc.flags, n, W, cp, mp, alpha,
                                           beta, _ptr(out))
    if rc:
        raise ValueError("oracle dequantize_accumulate: invalid arguments")
    return out


def _offsets(offsets, n: int) -> np.ndarray:
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    if off.ndim != 1 or off.size < 2:
        raise ValueError("layer offsets: need nl + 1 >= 2 entries")
    return off


def quantize_layers(desc: Desc, offsets, g, e=None, seed: int = 0,
                    step: int = 0):
    """Per-layer scale (TernGrad): layer l = g[off[l]:off[l+1]] is one bucket
    of the uniform scheme.  Returns (codes u8, meta f32[nl], e_new or None).
    desc.d is not used."""
    g = _f32(g)
    n = g.size
    off = _offsets(offsets, n)
    nl = off.size - 1
    e_new = None if e is None else _f32(e).copy()
    codes = np.zeros(desc.code_bytes(n), dtype=np.uint8)
    meta = np.zeros(nl, dtype=np.float32)
    rc = lib().gqref_quantize_layers(desc.s, desc.flags, n, nl, _ptr(off),
                                     _ptr(g), _ptr(e_new), seed, step,
                                     _ptr(codes), _ptr(meta))
    if rc:
        raise ValueError("oracle quantize_layers: invalid arguments")
    return codes, meta, e_new


def dequantize_accumulate_layers(desc: Desc, offsets, n: int, codes_list,
                                 meta_list, alpha: float = 1.0,
                                 beta: float = 0.0, out=None):
    off = _offsets(offsets, n)
    W = len(codes_list)
    cl = [np.ascontiguousarray(c, dtype=np.uint8) for c in codes_list]
    ml = [_f32(m) for m in meta_list]
    out = np.zeros(n, dtype=np.float32) if out is None else _f32(out).copy()
    cp = (C.c_void_p * W)(*[c.ctypes.data for c in cl])
    mp = (C.c_void_p * W)(*[m.ctypes.data for m in ml])
    rc = lib().gqref_dequantize_accumulate_layers(
        desc.s, desc.flags, n, off.size - 1, _ptr(off), W, cp, mp, alpha,
        beta, _ptr(out))
    if rc:
        raise ValueError("oracle dequantize_accumulate_layers: invalid arguments")
    return out


def topk_record_words(d: int, s: int, K: int) -> int:
    return lib().gqref_topk_record_words(d, s, K)


def quantize_topk(d: int, s: int, K: int, g, e=None, seed: int = 0,
                  step: int = 0, flags: int = 0):
    """Top-K + uniform quantization per bucket.  Returns (codes u8, meta
    f32[nb], e_new or None)."""
    g = _f32(g)
    n = g.size
    R = topk_record_words(d, s, K)
    if R < 0:
        raise ValueError("oracle quantize_topk: invalid arguments")
    nb = (n + d - 1) // d
    e_new = None if e is None else _f32(e).copy()
    codes = np.zeros(nb * R * 4, dtype=np.uint8)
    meta = np.zeros(nb, dtype=np.float32)
    rc = lib().gqref_quantize_topk(d, s, K, flags, n, _ptr(g), _ptr(e_new),
                                   seed, step, _ptr(codes), _ptr(meta))
    if rc:
        raise ValueError("oracle quantize_topk: invalid arguments")
    return codes, meta, e_new


def dequantize_accumulate_topk(d: int, s: int, K: int, n: int, codes_list,
                               meta_list, alpha: float = 1.0,
                               beta: float = 0.0, out=None, flags: int = 0):
    W = len(codes_list)
    cl = [np.ascontiguousarray(c, dtype=np.uint8) for c in codes_list]
    ml = [_f32(m) for m in meta_list]
    out = np.zeros(n, dtype=np.float32) if out is None else _f32(out).copy()
    cp = (C.c_void_p * W)(*[c.ctypes.data for c in cl])
    mp = (C.c_void_p * W)(*[m.ctypes.data for m in ml])
    rc = lib().gqref_dequantize_accumulate_topk(d, s, K, flags, n, W, cp, mp,
                                                alpha, beta, _ptr(out))
    if rc:
        raise ValueError("oracle dequantize_accumulate_topk: invalid arguments")
    return out


def pack(bits: int, vals) -> np.ndarray:
    v = np.ascontiguousarray(vals, dtype=np.uint32)
    out = np.zeros((v.size * bits + 7) // 8, dtype=np.uint8)
    lib().gqref_pack(bits, v.size, _ptr(v), _ptr(out))
    return out


def unpack(bits: int, n: int, codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(n, dtype=np.uint32)
    lib().gqref_unpack(bits, n, _ptr(c), _ptr(out))
    return out


def dense_width(A: int) -> int:
    return lib().gqref_dense_width(A)


def pack_dense(A: int, digits) -> np.ndarray:
    v = np.ascontiguousarray(digits, dtype=np.uint32)
    out = np.zeros((((v.size + 7) // 8) * dense_width(A) + 7) // 8, dtype=np.uint8)
    lib().gqref_pack_dense(A, v.size, _ptr(v), _ptr(out))
    return out


def unpack_dense(A: int, n: int, codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(n, dtype=np.uint32)
    lib().gqref_unpack_dense(A, n, _ptr(c), _ptr(out))
    return out


def signed_codes(desc: Desc, n: int, codes) -> np.ndarray:
    """Codes as integers: -s..s for the uniform scheme (two's complement or
    dense digits decoded), level index otherwise."""
    if desc.dense:
        v = unpack_dense(desc.alphabet, n, codes).astype(np.int64)
        return v - desc.s if desc.scheme == UNIFORM else v
    v = unpack(desc.bits, n, codes).astype(np.int64)
    if desc.scheme == UNIFORM:
        m = 1 << (desc.bits - 1)
        v = (v ^ m) - m
    return v


def elias_max_words(d: int, s: int, n: int) -> int:
    return int(lib().gqref_elias_max_words(d, s, n))


def elias_encode(d: int, s: int, n: int, codes):
    """Elias gamma stream of n uniform-scheme codes (fixed-width stream, s
    levels per sign).  Returns (off u64[nb + 1], words u32[off[nb]])."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    nb = (n + d - 1) // d
    off = np.zeros(nb + 1, dtype=np.uint64)
    if lib().gqref_elias_encode(d, s, n, _ptr(codes), _ptr(off), None):
        raise ValueError("oracle elias_encode: invalid arguments or codes")
    words = np.zeros(max(int(off[-1]), 1), dtype=np.uint32)
    if lib().gqref_elias_encode(d, s, n, _ptr(codes), _ptr(off), _ptr(words)):
        raise ValueError("oracle elias_encode: invalid arguments or codes")
    return off, words[:int(off[-1])]


def elias_decode(d: int, s: int, n: int, off, words):
    """Fixed-width codes (ceil(n * bits / 8) bytes) back from an Elias stream."""
    off = np.ascontiguousarray(off, dtype=np.uint64)
    words = np.ascontiguousarray(words, dtype=np.uint32)
    if words.size == 0:
        words = np.zeros(1, dtype=np.uint32)
    b = lib().gqref_bits(UNIFORM, s, 2)
    if b < 0:
        raise ValueError("oracle elias_decode: invalid arguments")
    codes = np.zeros((n * b + 7) // 8, dtype=np.uint8)
    if lib().gqref_elias_decode(d, s, n, _ptr(off), _ptr(words), _ptr(codes)):
        raise ValueError("oracle elias_decode: invalid arguments or stream")
    return codes


# ------------------------------------------------ layer-wise bit allocation --
# "Gradient Quantization" glossary, layer-wise quantization paragraph: layers
# with larger gradient variance get wider codes; the page gives no rule.
# Reading: widths b in {2, 3, 4, 8} with s = 2^(b-1) - 1 levels per sign on
# the per-layer scale path (the most a b-bit two's-complement code holds
# symmetrically); the objective is the sum over layers of the bound
# n_l * M_l^2 / (4 s_l^2) on the layer's rounding variance (every element's
# (b - x)(x - a) is at most step^2 / 4, step = M_l / s_l); every layer starts
# at 2 bits and upgrades are taken in decreasing order of bound reduction per
# added bit, M_l^2 (1/s_b^2 - 1/s_b'^2) / (4 (b' - b)), equal reductions by
# layer then width, until the first that does not fit the budget of code
# bits; upgrades that reduce nothing (M_l = 0, empty layers) are not taken.
# Parity status: pinned by brute force over every allocation of small
# layouts (the greedy's bound is the least of all allocations using no more
# bits), monotonicity in M_l, budget and extremes (tests/test_oracle_alloc).
ALLOC_WIDTHS = (2, 3, 4, 8)


def alloc_levels(bits: int) -> int:
    """s for a width b of the allocation: 2^(b-1) - 1."""
    return (1 << (bits - 1)) - 1


def alloc_gain_per_bit(scale: float, b0: int, b1: int) -> float:
    """Bound reduction per added code bit of one element when a layer of
    max-abs `scale` goes from b0 to b1 bits (fp64; the element count
    cancels)."""
    s0, s1 = alloc_levels(b0), alloc_levels(b1)
    m2 = float(np.float64(np.float32(scale))) ** 2
    return m2 * ((1.0 / (s0 * s0) - 1.0 / (s1 * s1)) / (4.0 * (b1 - b0)))


def allocate_layer_bits(sizes, scales, budget_bits: int):
    """Code width of every layer under a budget of total code bits.

    sizes: element count n_l of each layer; scales: its max-abs M_l (fp32);
    budget_bits: at least 2 * sum(sizes).  Returns (widths, bits used)."""
    sizes = [int(x) for x in sizes]
    nl = len(sizes)
    if len(scales) != nl or any(x < 0 for x in sizes):
        raise ValueError("allocate_layer_bits: sizes and scales differ")
    used = 2 * sum(sizes)
    if budget_bits < used:
        raise ValueError("allocate_layer_bits: budget below 2 bits per element")
    widths = [2] * nl
    ups = []
    for lay in range(nl):
        for b0, b1 in zip(ALLOC_WIDTHS[:-1], ALLOC_WIDTHS[1:]):
            ups.append((alloc_gain_per_bit(scales[lay], b0, b1), lay, b0, b1))
    ups.sort(key=lambda t: (-t[0], t[1], t[2]))
    for gain, lay, b0, b1 in ups:
        if gain <= 0.0:
            break  # the rest reduce nothing either
        if sizes[lay] == 0:
            continue
        cost = sizes[lay] * (b1 - b0)
        if used + cost > budget_bits:
            break
        assert widths[lay] == b0  # a layer's gains per bit strictly decrease
        widths[lay] = b1
        used += cost
    return widths, used


def alloc_segments(sizes, widths):
    """Byte offsets of the layers' code segments in a payload of the
    allocation: layer l's n_l codes LSB-first at widths[l] bits, each segment
    padded to a multiple of 16 bytes; the last entry is the payload size."""
    seg = [0]
    for n_l, b in zip(sizes, widths):
        nbytes = (int(n_l) * int(b) + 7) // 8
        seg.append(seg[-1] + (nbytes + 15) // 16 * 16)
    return seg


def quantize_layers_alloc(offsets, g, e, widths, seed: int = 0, step: int = 0,
                          flags: int = 0):
    """The per-layer scale path with layer l at widths[l] bits: each layer's
    codes are those quantize_layers gives at s = 2^(b-1) - 1 (same scale,
    random word and rounding), stored in the layer's own segment.  Returns
    (payload u8, meta f32[nl] = the layers' max-abs, e_new or None)."""
    g = _f32(g)
    n = g.size
    off = _offsets(offsets, n)
    nl = off.size - 1
    if len(widths) != nl or any(b not in ALLOC_WIDTHS for b in widths):
        raise ValueError("quantize_layers_alloc: one width from ALLOC_WIDTHS per layer")
    sizes = np.diff(off)
    seg = alloc_segments(sizes, widths)
    payload = np.zeros(seg[-1], dtype=np.uint8)
    e_new = None if e is None else np.empty(n, dtype=np.float32)
    meta = np.zeros(nl, dtype=np.float32)
    for b in sorted(set(widths)):
        d = Desc(UNIFORM, 512, s=alloc_levels(b), flags=flags)
        codes, m, en = quantize_layers(d, off, g, e, seed=seed, step=step)
        fields = unpack(b, n, codes)
        for lay in range(nl):
            if widths[lay] != b:
                continue
            lo, hi = int(off[lay]), int(off[lay + 1])
            meta[lay] = m[lay]
            if hi > lo:
                packed = pack(b, fields[lo:hi])
                payload[seg[lay]:seg[lay] + packed.size] = packed
            if e is not None:
                e_new[lo:hi] = en[lo:hi]
    return payload, meta, e_new


def dequantize_layers_alloc(offsets, n: int, payload, meta, widths):
    """x_hat of one allocation payload: each layer's codes times its step
    M_l / s_l, as dequantize_accumulate_layers gives at that layer's s."""
    off = _offsets(offsets, n)
    nl = off.size - 1
    sizes = np.diff(off)
    seg = alloc_segments(sizes, widths)
    pay = np.ascontiguousarray(payload, dtype=np.uint8)
    x = np.zeros(n, dtype=np.float32)
    for b in sorted(set(widths)):
        fields = np.zeros(n, dtype=np.uint32)
        for lay in range(nl):
            lo, hi = int(off[lay]), int(off[lay + 1])
            if widths[lay] == b and hi > lo:
                fields[lo:hi] = unpack(b, hi - lo, pay[seg[lay]:seg[lay + 1]])
        d = Desc(UNIFORM, 512, s=alloc_levels(b))
        xb = dequantize_accumulate_layers(d, off, n, [pack(b, fields)], [meta])
        for lay in range(nl):
            if widths[lay] == b:
                x[int(off[lay]):int(off[lay + 1])] = xb[int(off[lay]):int(off[lay + 1])]
    return x


def dequantize_accumulate_layers_alloc(offsets, n: int, payloads, metas,
                                       widths_list, alpha: float = 1.0,
                                       beta: float = 0.0, out=None):
    """out <- beta * out + alpha * sum_w x_hat_w over W allocation payloads
    (each with its own widths), summed in fp64 and rounded once."""
    acc = np.zeros(n, dtype=np.float64)
    for pay, m, wd in zip(payloads, metas, widths_list):
        acc += dequantize_layers_alloc(offsets, n, pay, m, wd).astype(np.float64)
    base = np.zeros(n) if out is None else _f32(out).astype(np.float64)
    return (float(beta) * base + float(alpha) * acc).astype(np.float32)
