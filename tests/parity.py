"""Helpers for GPU-vs-oracle parity tests (element-by-element comparison).

The tolerances are the stated ones:
  * codes / packed bytes: bit-exact (uniform, ternary, INT8, sign split),
    and for the sorted schemes bit-exact outside buckets the oracle records
    as near-ties;
  * meta: bit-exact for uniform; within 1e-5 relative for the two-level and
    ORQ levels (exact for unclipped ORQ outside ties, since its levels are
    input values);
  * dequantized values and residuals: within 1e-6 * max(|p|, |xhat|) (plus the
    level tolerance where a level differs), bit-exact expected for uniform;
  * aggregates: |d| <= 1e-6 * (|beta*out| + |alpha| * sum_w |xhat_w|).
"""
from __future__ import annotations

import sys

import numpy as np

import oracle as O

META_REL = 1e-5
VAL_REL = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bucket_code_bytes(desc: O.Desc) -> int:
    if desc.dense:
        return (desc.d // 8) * desc.field_bits // 8
    return desc.d * desc.bits // 8


def compare_codes(desc: O.Desc, n: int, got: np.ndarray, ref: np.ndarray,
                  tie: np.ndarray | None = None, exact: bool = True):
    """Compare packed codes bucket by bucket; returns the mismatching bucket
    indices (asserting they are all recorded ties unless exact)."""
    cb = desc.code_bytes(n)
    got = np.asarray(got[:cb])
    ref = np.asarray(ref[:cb])
    if np.array_equal(got, ref):
        return np.array([], dtype=np.int64)
    bpb = bucket_code_bytes(desc)
    bad = np.unique(np.nonzero(got != ref)[0] // bpb)
    if exact or tie is None:
        raise AssertionError(f"codes differ in buckets {bad[:20]} (of {bad.size})")
    untied = bad[tie[bad] == 0]
    assert untied.size == 0, f"codes differ outside recorded ties: {untied[:20]}"
    return bad


def compare_meta(desc: O.Desc, got: np.ndarray, ref: np.ndarray,
                 skip: np.ndarray | None = None, exact: bool = False):
    got = np.asarray(got, dtype=np.float32).reshape(ref.shape)
    if exact:
        assert np.array_equal(got, ref), _first_diff(got, ref)
        return
    mask = np.ones(ref.shape[0], dtype=bool)
    if skip is not None and skip.size:
        mask[skip] = False
    g, r = got[mask].astype(np.float64), ref[mask].astype(np.float64)
    err = np.abs(g - r)
    tol = META_REL * np.abs(r)
    assert np.all(err <= tol), _first_diff(got[mask], ref[mask])


def compare_values(got: np.ndarray, ref: np.ndarray, scale: np.ndarray,
                   exact: bool = False, extra: np.ndarray | float = 0.0):
    if exact:
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
            _first_diff(got, ref)
        return
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    tol = VAL_REL * scale + extra
    assert np.all(err <= tol), _first_diff(got, ref)


def _first_diff(got, ref):
    g = np.asarray(got).ravel()
    r = np.asarray(ref).ravel()
    idx = np.nonzero(g != r)[0]
    if idx.size == 0:
        return "no difference"
    i = idx[0]
    return f"{idx.size} differences, first at {i}: got {g[i]!r} ref {r[i]!r}"


def bucket_mask(desc: O.Desc, n: int, buckets: np.ndarray) -> np.ndarray:
    m = np.ones(n, dtype=bool)
    for b in buckets:
        m[b * desc.d: min(n, (b + 1) * desc.d)] = False
    return m


def sample_runs(nb: int, runs: int, run_len: int, seed: int = 0):
    """Start buckets of `runs` runs of `run_len` consecutive buckets, always
    including the first and the last bucket."""
    rng = np.random.default_rng(seed)
    starts = set([0, max(0, nb - run_len)])
    if nb > run_len:
        starts.update(rng.integers(0, nb - run_len, runs).tolist())
    return sorted(starts)
