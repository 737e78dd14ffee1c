"""Python binding of libgq (include/gq.h): argument marshalling only.

Every entry point has the C name and forwards device pointers from PyTorch
tensors (PyTorch supplies device memory and the current HIP stream; all
arithmetic runs in libgq's HIP kernels).  Importing this module loads the
in-tree ``libgq.so`` and raises if it has not been built: there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgq.so")

GQ_UNIFORM, GQ_BIN_SIGN, GQ_BIN_OPT, GQ_ORQ, GQ_TOPK = 0, 1, 2, 3, 4
GQ_FLAG_CLIP = 1
GQ_FLAG_DENSE = 2
GQ_FLAG_NEAREST = 4
GQ_FLAG_BISECT = 8
GQ_OK, GQ_EINVAL, GQ_EUNSUPPORTED, GQ_ELAUNCH, GQ_ETOOMANY = 0, -1, -2, -3, -4
GQ_MAX_PAYLOADS = 16

SYMBOLS = ("gq_code_bits", "gq_payload_size", "gq_select_levels",
           "gq_quantize", "gq_error_feedback", "gq_dequantize_accumulate",
           "gq_quantize_layers", "gq_dequantize_accumulate_layers",
           "gq_allocate_layer_bits", "gq_alloc_payload_bytes",
           "gq_quantize_layers_alloc", "gq_dequantize_accumulate_layers_alloc",
           "gq_elias_max_words", "gq_elias_encode", "gq_elias_decode",
           "gq_strerror", "gq_version")


class gq_desc(C.Structure):
    _fields_ = [("scheme", C.c_int32), ("bucket", C.c_int32), ("s", C.c_int32),
                ("levels", C.c_int32), ("flags", C.c_int32),
                ("clip_sigma", C.c_float)]

    def __repr__(self) -> str:
        return (f"gq_desc(scheme={self.scheme}, bucket={self.bucket}, s={self.s}, "
                f"levels={self.levels}, flags={self.flags}, "
                f"clip_sigma={self.clip_sigma})")


class GQError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {gq_strerror(status)} (status {status})")
        self.status = status


def _load():
    # GQ_LIBRARY: load another build of the same sources instead (the host
    # sanitizer test loads an AddressSanitizer build of the C ABI this way)
    path = os.environ.get("GQ_LIBRARY", LIB_PATH)
    if not os.path.exists(path):
        raise ImportError(
            f"libgq.so not found at {path}; build it with "
            "`python -m communication_efficient_gradient_amd.build`")
    lib = C.CDLL(path)
    P = C.c_void_p
    D = C.POINTER(gq_desc)
    i64, i32 = C.c_int64, C.c_int32
    lib.gq_code_bits.argtypes = [D, C.POINTER(i32)]
    lib.gq_payload_size.argtypes = [D, i64, C.POINTER(i64), C.POINTER(i64)]
    lib.gq_select_levels.argtypes = [D, i64, P, P, P, P]
    lib.gq_quantize.argtypes = [D, i64, P, P, C.c_uint64, C.c_uint32, P, P, P]
    lib.gq_error_feedback.argtypes = [D, i64, P, P, P, P, P]
    lib.gq_dequantize_accumulate.argtypes = [D, i64, i32, C.POINTER(P),
                                             C.POINTER(P), C.c_float,
                                             C.c_float, P, P]
    lib.gq_quantize_layers.argtypes = [D, i64, i32, P, P, P, C.c_uint64,
                                       C.c_uint32, P, P, P]
    lib.gq_dequantize_accumulate_layers.argtypes = [
        D, i64, i32, P, i32, C.POINTER(P), C.POINTER(P), C.c_float, C.c_float,
        P, P]
    lib.gq_allocate_layer_bits.argtypes = [i64, i32, P, P, i64, P, P, P]
    lib.gq_alloc_payload_bytes.argtypes = [i64, i32, C.POINTER(i64)]
    lib.gq_quantize_layers_alloc.argtypes = [i64, i32, P, P, P, P, P, C.c_uint64,
                                             C.c_uint32, i32, P, i64, P, P]
    lib.gq_dequantize_accumulate_layers_alloc.argtypes = [
        i64, i32, P, i32, C.POINTER(P), C.POINTER(P), C.POINTER(P),
        C.POINTER(P), C.c_float, C.c_float, P, P]
    lib.gq_elias_max_words.argtypes = [D, i64, C.POINTER(i64)]
    lib.gq_elias_encode.argtypes = [D, i64, P, P, P, P]
    lib.gq_elias_decode.argtypes = [D, i64, P, P, i64, P, P]
    lib.gq_strerror.argtypes = [C.c_int]
    lib.gq_strerror.restype = C.c_char_p
    lib.gq_version.argtypes = []
    for name in SYMBOLS:
        if name not in ("gq_strerror",):
            getattr(lib, name).restype = C.c_int
    return lib


_lib = _load()


def lib():
    return _lib


def desc(scheme: int = GQ_UNIFORM, bucket: int = 512, s: int = 4,
         levels: int = 5, flags: int = 0, clip_sigma: float = 3.0) -> gq_desc:
    return gq_desc(scheme, bucket, s, levels, flags, clip_sigma)


def gq_strerror(status: int) -> str:
    return _lib.gq_strerror(status).decode()


def gq_version() -> int:
    return _lib.gq_version()


def _check(status: int, what: str) -> None:
    if status != GQ_OK:
        raise GQError(status, what)


def gq_code_bits(d: gq_desc) -> int:
    b = C.c_int32()
    _check(_lib.gq_code_bits(C.byref(d), C.byref(b)), "gq_code_bits")
    return b.value


def gq_payload_size(d: gq_desc, n: int):
    """Returns (code_bytes, code_capacity, meta_floats); code_capacity is
    code_bytes rounded up to a multiple of 16, the size of a codes buffer
    that gq_quantize writes."""
    cb, mf = C.c_int64(), C.c_int64()
    _check(_lib.gq_payload_size(C.byref(d), n, C.byref(cb), C.byref(mf)),
           "gq_payload_size")
    return cb.value, (cb.value + 15) // 16 * 16, mf.value


def _ptr(t, dtype, what):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    return t.data_ptr()


def _stream(stream, ref: torch.Tensor):
    if stream is None:
        return torch.cuda.current_stream(ref.device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def alloc_payload(d: gq_desc, n: int, device="cuda"):
    """Device buffers for one payload: (codes u8[code_capacity], meta f32)."""
    _, cap, mf = gq_payload_size(d, n)
    codes = torch.empty(cap, dtype=torch.uint8, device=device)
    meta = torch.empty(mf, dtype=torch.float32, device=device)
    return codes, meta


def _need(t: torch.Tensor, count: int, what: str) -> None:
    if t.numel() < count:
        raise ValueError(f"{what}: needs {count} elements, has {t.numel()}")


def gq_select_levels(d: gq_desc, g: torch.Tensor, e: torch.Tensor | None,
                     meta: torch.Tensor, stream=None) -> None:
    _, _, mf = gq_payload_size(d, g.numel())
    _need(meta, mf, "meta")
    if e is not None and e.numel() != g.numel():
        raise ValueError("e must have g's size")
    _check(_lib.gq_select_levels(
        C.byref(d), g.numel(), _ptr(g, torch.float32, "g"),
        _ptr(e, torch.float32, "e"), _ptr(meta, torch.float32, "meta"),
        _stream(stream, g)), "gq_select_levels")


def gq_quantize(d: gq_desc, g: torch.Tensor, e: torch.Tensor | None,
                seed: int, step: int, codes: torch.Tensor, meta: torch.Tensor,
                stream=None) -> None:
    if e is not None and e.numel() != g.numel():
        raise ValueError("e must have g's size")
    _, cap, mf = gq_payload_size(d, g.numel())
    _need(codes, cap, "codes")
    _need(meta, mf, "meta")
    _check(_lib.gq_quantize(
        C.byref(d), g.numel(), _ptr(g, torch.float32, "g"),
        _ptr(e, torch.float32, "e"), seed, step,
        _ptr(codes, torch.uint8, "codes"), _ptr(meta, torch.float32, "meta"),
        _stream(stream, g)), "gq_quantize")


def gq_error_feedback(d: gq_desc, g: torch.Tensor, e: torch.Tensor,
                      codes: torch.Tensor, meta: torch.Tensor,
                      stream=None) -> None:
    if e.numel() != g.numel():
        raise ValueError("e must have g's size")
    cb, _, mf = gq_payload_size(d, g.numel())
    _need(codes, cb, "codes")
    _need(meta, mf, "meta")
    _check(_lib.gq_error_feedback(
        C.byref(d), g.numel(), _ptr(g, torch.float32, "g"),
        _ptr(e, torch.float32, "e"), _ptr(codes, torch.uint8, "codes"),
        _ptr(meta, torch.float32, "meta"), _stream(stream, g)),
        "gq_error_feedback")


def gq_dequantize_accumulate(d: gq_desc, n: int,
                             codes: Sequence[torch.Tensor],
                             meta: Sequence[torch.Tensor], alpha: float,
                             beta: float, out: torch.Tensor,
                             stream=None) -> None:
    W = len(codes)
    if len(meta) != W:
        raise ValueError("codes and meta must have the same length")
    if out.numel() < n:
        raise ValueError("out is smaller than n")
    if 1 <= W <= GQ_MAX_PAYLOADS:
        cb, _, mf = gq_payload_size(d, n)
        for c, m in zip(codes, meta):
            _need(c, cb, "codes")
            _need(m, mf, "meta")
    cp = (C.c_void_p * max(W, 1))(*[_ptr(c, torch.uint8, "codes") for c in codes])
    mp = (C.c_void_p * max(W, 1))(*[_ptr(m, torch.float32, "meta") for m in meta])
    _check(_lib.gq_dequantize_accumulate(
        C.byref(d), n, W, cp, mp, alpha, beta, _ptr(out, torch.float32, "out"),
        _stream(stream, out)), "gq_dequantize_accumulate")


def _offsets(off: torch.Tensor) -> int:
    if off.dim() != 1 or off.numel() < 2:
        raise ValueError("layer_offsets: a 1-D tensor of nl + 1 >= 2 entries")
    return _ptr(off, torch.int64, "layer_offsets")


def gq_quantize_layers(d: gq_desc, layer_offsets: torch.Tensor,
                       g: torch.Tensor, e: torch.Tensor | None, seed: int,
                       step: int, codes: torch.Tensor, meta: torch.Tensor,
                       stream=None) -> None:
    """Per-layer scale: layer_offsets is an int64 device tensor of nl + 1
    flat offsets; meta receives nl floats."""
    if e is not None and e.numel() != g.numel():
        raise ValueError("e must have g's size")
    op = _offsets(layer_offsets)
    nl = layer_offsets.numel() - 1
    _, cap, _ = gq_payload_size(d, g.numel())
    _need(codes, cap, "codes")
    _need(meta, nl, "meta")
    _check(_lib.gq_quantize_layers(
        C.byref(d), g.numel(), nl, op, _ptr(g, torch.float32, "g"),
        _ptr(e, torch.float32, "e"), seed, step,
        _ptr(codes, torch.uint8, "codes"), _ptr(meta, torch.float32, "meta"),
        _stream(stream, g)), "gq_quantize_layers")


def gq_dequantize_accumulate_layers(d: gq_desc, n: int,
                                    layer_offsets: torch.Tensor,
                                    codes: Sequence[torch.Tensor],
                                    meta: Sequence[torch.Tensor],
                                    alpha: float, beta: float,
                                    out: torch.Tensor, stream=None) -> None:
    W = len(codes)
    if len(meta) != W:
        raise ValueError("codes and meta must have the same length")
    if out.numel() < n:
        raise ValueError("out is smaller than n")
    op = _offsets(layer_offsets)
    nl = layer_offsets.numel() - 1
    if 1 <= W <= GQ_MAX_PAYLOADS:
        cb, _, _ = gq_payload_size(d, n)
        for c, m in zip(codes, meta):
            _need(c, cb, "codes")
            _need(m, nl, "meta")
    cp = (C.c_void_p * max(W, 1))(*[_ptr(c, torch.uint8, "codes") for c in codes])
    mp = (C.c_void_p * max(W, 1))(*[_ptr(m, torch.float32, "meta") for m in meta])
    _check(_lib.gq_dequantize_accumulate_layers(
        C.byref(d), n, nl, op, W, cp, mp, alpha, beta,
        _ptr(out, torch.float32, "out"), _stream(stream, out)),
        "gq_dequantize_accumulate_layers")


# ---------------------------------------------------------------------------
# Prepared calls: validate and marshal the arguments once, then re-issue the
# same launch with only (seed, step) changing.  For launch loops where the
# per-call Python checks above would otherwise dominate a ~10 us kernel.
def gq_elias_max_words(d: gq_desc, n: int) -> int:
    w = C.c_int64()
    _check(_lib.gq_elias_max_words(C.byref(d), n, C.byref(w)), "gq_elias_max_words")
    return w.value


def alloc_elias(d: gq_desc, n: int, device="cuda"):
    """Device buffers for one Elias stream: (offsets i64[nb + 1], words
    i32[gq_elias_max_words]); the bits are those of the C ABI's uint64 /
    uint32 arrays."""
    nb = (n + d.bucket - 1) // d.bucket
    off = torch.empty(nb + 1, dtype=torch.int64, device=device)
    words = torch.empty(max(gq_elias_max_words(d, n), 1), dtype=torch.int32,
                        device=device)
    return off, words


def gq_elias_encode(d: gq_desc, n: int, codes: torch.Tensor,
                    offsets: torch.Tensor, words: torch.Tensor,
                    stream=None) -> None:
    """Elias gamma stream of a gq_quantize payload's codes."""
    _, cap, _ = gq_payload_size(d, n)
    _need(codes, cap, "codes")
    _need(offsets, (n + d.bucket - 1) // d.bucket + 1, "offsets")
    _need(words, gq_elias_max_words(d, n), "words")
    _check(_lib.gq_elias_encode(
        C.byref(d), n, _ptr(codes, torch.uint8, "codes"),
        _ptr(offsets, torch.int64, "offsets"), _ptr(words, torch.int32, "words"),
        _stream(stream, codes)), "gq_elias_encode")


def gq_elias_decode(d: gq_desc, n: int, offsets: torch.Tensor,
                    words: torch.Tensor, codes: torch.Tensor,
                    n_words: int | None = None, stream=None) -> None:
    """Fixed-width codes back from an Elias stream (n_words: the readable
    length of words, default its size)."""
    _, cap, _ = gq_payload_size(d, n)
    _need(codes, cap, "codes")
    _need(offsets, (n + d.bucket - 1) // d.bucket + 1, "offsets")
    nw = words.numel() if n_words is None else int(n_words)
    if nw > words.numel():
        raise ValueError("n_words exceeds the words tensor")
    _check(_lib.gq_elias_decode(
        C.byref(d), n, _ptr(offsets, torch.int64, "offsets"),
        _ptr(words, torch.int32, "words"), nw, _ptr(codes, torch.uint8, "codes"),
        _stream(stream, codes)), "gq_elias_decode")


class PreparedQuantize:
    def __init__(self, d: gq_desc, g: torch.Tensor, e: torch.Tensor | None,
                 codes: torch.Tensor, meta: torch.Tensor, stream=None):
        if e is not None and e.numel() != g.numel():
            raise ValueError("e must have g's size")
        _, cap, mf = gq_payload_size(d, g.numel())
        _need(codes, cap, "codes")
        _need(meta, mf, "meta")
        self._keep = (d, g, e, codes, meta)
        self._args = (C.byref(d), g.numel(), _ptr(g, torch.float32, "g"),
                      _ptr(e, torch.float32, "e"))
        self._tail = (_ptr(codes, torch.uint8, "codes"),
                      _ptr(meta, torch.float32, "meta"), _stream(stream, g))

    def __call__(self, seed: int, step: int) -> None:
        _check(_lib.gq_quantize(*self._args, seed, step, *self._tail),
               "gq_quantize")


class PreparedDequantizeAccumulate:
    def __init__(self, d: gq_desc, n: int, codes: Sequence[torch.Tensor],
                 meta: Sequence[torch.Tensor], alpha: float, beta: float,
                 out: torch.Tensor, stream=None):
        W = len(codes)
        if len(meta) != W or not 1 <= W <= GQ_MAX_PAYLOADS:
            raise ValueError("need 1..GQ_MAX_PAYLOADS (codes, meta) pairs")
        if out.numel() < n:
            raise ValueError("out is smaller than n")
        cb, _, mf = gq_payload_size(d, n)
        for c, m in zip(codes, meta):
            _need(c, cb, "codes")
            _need(m, mf, "meta")
        self._keep = (d, list(codes), list(meta), out)
        cp = (C.c_void_p * W)(*[_ptr(c, torch.uint8, "codes") for c in codes])
        mp = (C.c_void_p * W)(*[_ptr(m, torch.float32, "meta") for m in meta])
        self._ptrs = (cp, mp)
        self._args = (C.byref(d), n, W, cp, mp, alpha, beta,
                      _ptr(out, torch.float32, "out"), _stream(stream, out))

    def __call__(self) -> None:
        _check(_lib.gq_dequantize_accumulate(*self._args),
               "gq_dequantize_accumulate")


def gq_allocate_layer_bits(n: int, layer_offsets: torch.Tensor,
                           scales: torch.Tensor, budget_bits: int,
                           widths: torch.Tensor, segments: torch.Tensor,
                           stream=None) -> None:
    """Widths (int32[nl]) and code segment offsets (int64[nl + 1]) of the
    layer-wise allocation; see include/gq.h."""
    nl = layer_offsets.numel() - 1
    _need(scales, nl, "scales")
    _need(widths, nl, "widths")
    _need(segments, nl + 1, "segments")
    _check(_lib.gq_allocate_layer_bits(
        n, nl, _ptr(layer_offsets, torch.int64, "layer_offsets"),
        _ptr(scales, torch.float32, "scales"), budget_bits,
        _ptr(widths, torch.int32, "widths"), _ptr(segments, torch.int64, "segments"),
        _stream(stream, scales)), "gq_allocate_layer_bits")


def gq_alloc_payload_bytes(n: int, nl: int) -> int:
    """Bytes a payload of any layer-wise allocation of n elements in nl
    layers needs (n + 16 nl)."""
    b = C.c_int64(0)
    _check(_lib.gq_alloc_payload_bytes(n, nl, C.byref(b)), "gq_alloc_payload_bytes")
    return b.value


def gq_quantize_layers_alloc(layer_offsets: torch.Tensor, g: torch.Tensor,
                             e: torch.Tensor | None, widths: torch.Tensor,
                             segments: torch.Tensor, seed: int, step: int,
                             payload: torch.Tensor, meta: torch.Tensor,
                             flags: int = 0, stream=None) -> None:
    """Codes of each layer at its allocated width in its own segment (and
    the residual); see include/gq.h."""
    n = g.numel()
    nl = layer_offsets.numel() - 1
    if e is not None and e.numel() != n:
        raise ValueError("e and g differ in size")
    _need(widths, nl, "widths")
    _need(segments, nl + 1, "segments")
    _need(meta, nl, "meta")
    _check(_lib.gq_quantize_layers_alloc(
        n, nl, _offsets(layer_offsets), _ptr(g, torch.float32, "g"),
        _ptr(e, torch.float32, "e"), _ptr(widths, torch.int32, "widths"),
        _ptr(segments, torch.int64, "segments"), seed, step, flags,
        _ptr(payload, torch.uint8, "payload"), payload.numel(),
        _ptr(meta, torch.float32, "meta"), _stream(stream, g)),
        "gq_quantize_layers_alloc")


def gq_dequantize_accumulate_layers_alloc(n: int, layer_offsets: torch.Tensor,
                                          payloads: Sequence[torch.Tensor],
                                          meta: Sequence[torch.Tensor],
                                          widths: Sequence[torch.Tensor],
                                          segments: Sequence[torch.Tensor],
                                          alpha: float, beta: float,
                                          out: torch.Tensor, stream=None) -> None:
    """out <- beta out + alpha sum of the payloads' x_hat; see include/gq.h."""
    W = len(payloads)
    if not (len(meta) == len(widths) == len(segments) == W):
        raise ValueError("payloads, meta, widths and segments differ in length")
    if out.numel() < n:
        raise ValueError("out is smaller than n")
    nl = layer_offsets.numel() - 1
    for m, wd, sg in zip(meta, widths, segments):
        _need(m, nl, "meta")
        _need(wd, nl, "widths")
        _need(sg, nl + 1, "segments")

    def arr(ts, dt, what):
        return (C.c_void_p * max(W, 1))(*[_ptr(t, dt, what) for t in ts])

    _check(_lib.gq_dequantize_accumulate_layers_alloc(
        n, nl, _offsets(layer_offsets), W, arr(payloads, torch.uint8, "payload"),
        arr(meta, torch.float32, "meta"), arr(widths, torch.int32, "widths"),
        arr(segments, torch.int64, "segments"), alpha, beta,
        _ptr(out, torch.float32, "out"), _stream(stream, out)),
        "gq_dequantize_accumulate_layers_alloc")
