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
        if _build.needs_build():
            _build.build()
        L = C.CDLL(_build.LIB)
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
