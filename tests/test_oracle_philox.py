"""Pins for the oracle's Philox4x32-10 (counter-based RNG for random rounding).

The pages require rounding that is random and unbiased ("Gradient
Quantization" glossary, Stochastic Quantization bullet) but name no
generator; Philox4x32-10 (Salmon et al., SC'11) with key = seed and counter =
(i/4, step) is this build's choice.  Pinned against an independent
implementation (rocRAND, run on the host) and by statistics.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_words(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND pin")
    exe = str(tmp_path_factory.mktemp("pin") / "philox_pin")
    subprocess.run([hipcc, "-O1", os.path.join(HERE, "philox_rocrand_pin.cpp"),
                    "-o", exe], check=True, capture_output=True)

    def run(triples):
        inp = "".join(f"{s} {i} {t}\n" for s, i, t in triples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True,
                             check=True).stdout.split()
        return np.array([int(x) for x in out], dtype=np.uint64)

    return run


def test_philox_matches_rocrand(rocrand_words):
    rng = np.random.default_rng(7)
    triples = []
    for seed in [0, 1, 2, 3, 8, 0xFFFFFFFF, 0x1_0000_0001, 2**64 - 1]:
        for step in [0, 1, 4, 2**31 + 5]:
            for i in [0, 1, 2, 3, 4, 7, 511, 65535, 2**32 + 3,
                      4 * 2**32 + 2, 2**40 + 1]:
                triples.append((seed, i, step))
    for _ in range(200):
        triples.append((int(rng.integers(0, 2**63)), int(rng.integers(0, 2**42)),
                        int(rng.integers(0, 2**32))))
    ref = rocrand_words(triples)
    ours = np.array([O.philox(s, i // 4, t)[i % 4] for s, i, t in triples],
                    dtype=np.uint64)
    assert np.array_equal(ours, ref)


def test_philox_bit_frequencies_and_uniformity():
    # 2^22 blocks = 2^24 words: every bit position is 1 with probability 1/2
    words = O.philox_blocks(1234, 0, 1 << 22, 3).ravel()
    n = words.size
    bits = np.unpackbits(words.view(np.uint8)).reshape(n, 32).sum(axis=0)
    z = (bits - n / 2) / np.sqrt(n / 4)
    assert np.all(np.abs(z) < 6), z
    # 24-bit uniforms u = (w >> 8) 2^-24: chi-square over 256 equal bins
    u = (words >> 8).astype(np.float64) * 2.0**-24
    assert u.min() >= 0.0 and u.max() < 1.0
    counts = np.bincount((u * 256).astype(np.int64), minlength=256)
    exp = n / 256
    chi2 = ((counts - exp) ** 2 / exp).sum()
    # chi2(255): mean 255, sd ~22.6
    assert abs(chi2 - 255) < 6 * np.sqrt(2 * 255), chi2


def test_philox_streams_differ_by_seed_step_and_counter():
    a = O.philox_blocks(5, 0, 1024, 0)
    b = O.philox_blocks(6, 0, 1024, 0)
    c = O.philox_blocks(5, 0, 1024, 1)
    d = O.philox_blocks(5, 1, 1024, 0)
    assert np.array_equal(a[1:], d[:-1])
    for x, y in [(a, b), (a, c)]:
        assert (x != y).mean() > 0.99
