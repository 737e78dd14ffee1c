"""Seeded synthetic gradients for the five benchmark workloads.

This module only draws numbers: it holds none of the quantizer's arithmetic,
so the CPU oracle and the HIP library can both be fed from it.

The pages measure accuracy on CIFAR/ImageNet ("Optimal Gradient Quantization
Condition" review, §Key findings); no dataset is used here.  Each generator
below draws fp32 gradients with the distribution the workload names, in
2**24-element chunks, each chunk from its own ``numpy.random.default_rng``
seed sequence, so any chunk can be regenerated on its own and the result does
not depend on how many threads fill it.

Workloads (sizes decimal: M = 1e6, B = 1e9):

* ``qsgd``     65,536 elements, N(0, 1e-3^2)            (QSGD, s=4)
* ``ternary``  25.6M elements in 160 Laplace "layers"    (TernGrad + EF, 5 steps)
* ``orq``      100M elements, 0.9 N(0,1) + 0.1 t(3), x1e-3 (ORQ-5/9)
* ``bingrad``  1B elements, 0.7 N(0,1e-4^2) + 0.3 N(0,1e-2^2) (BinGrad-b + EF)
* ``workers``  8 x 256M elements, (shared + own) N(0,1) x 1e-3 (INT8 + EF, W=8)
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 24

QSGD_N = 65_536
TERNARY_N = 25_600_000
TERNARY_LAYERS = 160
TERNARY_STEPS = 5
ORQ_N = 100_000_000
BINGRAD_N = 1_000_000_000
WORKERS_N = 256_000_000
WORKERS_W = 8


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill_chunks(n: int, make_chunk, out: np.ndarray | None = None,
                 start: int = 0) -> np.ndarray:
    """Fill ``out[0:n]`` with elements ``start .. start+n`` of a chunked stream.

    ``make_chunk(k, m)`` returns the fp32 chunk ``k`` of length ``m``
    (every chunk but the last has ``CHUNK`` elements).  ``start`` must be a
    multiple of ``CHUNK``.
    """
    if start % CHUNK:
        raise ValueError("start must be a multiple of the chunk size")
    if out is None:
        out = np.empty(n, dtype=np.float32)
    k0 = start // CHUNK
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c: int) -> None:
        lo = c * CHUNK
        m = min(CHUNK, n - lo)
        out[lo:lo + m] = make_chunk(k0 + c, m)

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


# ---------------------------------------------------------------- qsgd ----
def qsgd_gradient(n: int = QSGD_N) -> np.ndarray:
    """N(0, 1e-3^2) fp32 from seed 0 (drawn in fp64, scaled, rounded once)."""
    x = np.random.default_rng([0, 0]).standard_normal(n)
    return (x * 1e-3).astype(np.float32)


# ------------------------------------------------------------- ternary ----
def ternary_layout(n: int = TERNARY_N, layers: int = TERNARY_LAYERS):
    """Layer sizes (log-uniform on [1024, 2.4M], rescaled to sum to ``n``)
    and per-layer Laplace scales (log-uniform on [1e-5, 1e-2])."""
    rng = np.random.default_rng(20)
    raw = np.exp(rng.uniform(np.log(1024.0), np.log(2.4e6), layers))
    scales = np.exp(rng.uniform(np.log(1e-5), np.log(1e-2), layers))
    sizes = np.floor(raw * (n / raw.sum())).astype(np.int64)
    sizes = np.maximum(sizes, 1)
    sizes[-1] = n - sizes[:-1].sum()
    if sizes[-1] < 1:
        raise ValueError("layer layout does not fit n")
    return sizes, scales


def ternary_gradient(step: int, n: int = TERNARY_N,
                     layers: int = TERNARY_LAYERS) -> np.ndarray:
    """Step ``step``: the layers' Laplace(0, b_l) draws concatenated flat."""
    sizes, scales = ternary_layout(n, layers)
    out = np.empty(n, dtype=np.float32)
    offs = np.concatenate([[0], np.cumsum(sizes)])

    def work(l: int) -> None:
        x = np.random.default_rng([21, step, l]).laplace(0.0, scales[l], sizes[l])
        out[offs[l]:offs[l + 1]] = x.astype(np.float32)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(layers)))
    return out


# ----------------------------------------------------------------- orq ----
def _orq_chunk(k: int, m: int) -> np.ndarray:
    rng = np.random.default_rng([3, k])
    z = rng.standard_normal(m)
    t = rng.standard_t(3, m)
    sel = rng.random(m) < 0.1
    return (np.where(sel, t, z) * 1e-3).astype(np.float32)


def orq_gradient(n: int = ORQ_N, out=None, start: int = 0) -> np.ndarray:
    """90 % N(0,1) / 10 % Student-t(3), per element, times 1e-3."""
    return _fill_chunks(n, _orq_chunk, out, start)


# ------------------------------------------------------------- bingrad ----
def _bingrad_chunk(k: int, m: int) -> np.ndarray:
    rng = np.random.default_rng([4, k])
    z = rng.standard_normal(m)
    sel = rng.random(m) < 0.7
    return (z * np.where(sel, 1e-4, 1e-2)).astype(np.float32)


def bingrad_gradient(n: int = BINGRAD_N, out=None, start: int = 0) -> np.ndarray:
    """Mixture 0.7 N(0, 1e-4^2) + 0.3 N(0, 1e-2^2)."""
    return _fill_chunks(n, _bingrad_chunk, out, start)


# ------------------------------------------------------------- workers ----
def worker_gradient(w: int, n: int = WORKERS_N, out=None,
                    start: int = 0) -> np.ndarray:
    """Worker ``w`` (1..8): (shared + own) standard normals times 1e-3; the
    shared part comes from seed 0, which no worker uses as its own."""
    if w < 1:
        raise ValueError("workers are numbered from 1")

    def chunk(k: int, m: int) -> np.ndarray:
        shared = np.random.default_rng([0, k]).standard_normal(m)
        own = np.random.default_rng([w, k]).standard_normal(m)
        return ((shared + own) * 1e-3).astype(np.float32)

    return _fill_chunks(n, chunk, out, start)


def small_mixture(n: int, seed: int, kind: str = "normal") -> np.ndarray:
    """Small seeded inputs for edge-case tests (not a benchmark workload)."""
    rng = np.random.default_rng([99, seed])
    if kind == "normal":
        x = rng.standard_normal(n) * 1e-3
    elif kind == "laplace":
        x = rng.laplace(0.0, 1e-3, n)
    elif kind == "heavy":
        x = rng.standard_t(2, n) * 1e-3
    elif kind == "wide":
        x = rng.standard_normal(n) * np.exp(rng.uniform(-30, 30, n))
    elif kind == "ints":
        x = rng.integers(-3, 4, n).astype(np.float64)
    elif kind == "positive":
        x = np.abs(rng.standard_normal(n)) + 1.0
    else:
        raise ValueError(kind)
    return x.astype(np.float32)


# ------------------------------------------------------------- digests ----
def chunk_sha256(x: np.ndarray) -> list:
    """SHA-256 of each CHUNK-element slice of ``x`` (fp32, little-endian
    bytes), so an input can be checked chunk by chunk."""
    import hashlib
    b = np.ascontiguousarray(x, dtype="<f4")
    return [hashlib.sha256(b[lo:lo + CHUNK].tobytes()).hexdigest()
            for lo in range(0, b.size, CHUNK)]


def all_digests() -> dict:
    """Chunk digests of every benchmark input at its full size (generated
    one at a time; about 4 GB at the largest)."""
    out = {"numpy": np.__version__, "chunk": CHUNK}
    out["qsgd"] = chunk_sha256(qsgd_gradient())
    out["ternary"] = [chunk_sha256(ternary_gradient(t)) for t in range(TERNARY_STEPS)]
    out["orq"] = chunk_sha256(orq_gradient())
    out["bingrad"] = chunk_sha256(bingrad_gradient())
    out["workers"] = [chunk_sha256(worker_gradient(w)) for w in range(1, WORKERS_W + 1)]
    return out


if __name__ == "__main__":
    # python -m communication_efficient_gradient_amd.workloads OUT.json
    import json
    import sys
    with open(sys.argv[1], "w") as f:
        json.dump(all_digests(), f, indent=1)
        f.write("\n")
