"""Pins of the oracle's Elias gamma coding of uniform-scheme codes (QSGD's
lossless integer coding: "Gradient Quantization" glossary, QSGD paragraph).

Reading under test: code c becomes gamma(|c| + 1) followed by a sign bit
(1 = negative) when c != 0; each bucket's record starts on a 32-bit word;
off[j] is record j's first word.

The pins: the textbook gamma codewords and a hand-written stream
(tests/golden/elias_gamma.json); a parser written here on strings of '0'/'1'
(independent of the oracle's reader) recovers every code; record lengths
from the code-length formula with Python's int.bit_length; the Shannon bound
(no uniquely decodable code of single symbols beats the empirical entropy);
round trips through the oracle's decoder; the worst case meets
elias_max_words; corrupt streams and out-of-range codes are rejected.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
from communication_efficient_gradient_amd import workloads as WL

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "elias_gamma.json")))


def _bits(words, n_words):
    """Stream bits as a '0'/'1' string, bit t = bit t mod 32 of word t / 32."""
    w = np.asarray(words, dtype=np.uint32)[:n_words]
    return "".join(map(str, np.unpackbits(w.view(np.uint8), bitorder="little")))


def _parse(bitstr, count):
    """count codes from a record's bit string, by string operations."""
    out, t = [], 0
    for _ in range(count):
        L = 0
        while bitstr[t] == "0":
            L += 1
            t += 1
        m = int(bitstr[t:t + L + 1], 2)
        t += L + 1
        c = m - 1
        if c:
            if bitstr[t] == "1":
                c = -c
            t += 1
        out.append(c)
    return out, t


def _codes(s, vals):
    b = O.Desc(O.UNIFORM, 64, s=s).bits
    return O.pack(b, np.asarray(vals, dtype=np.int64) & ((1 << b) - 1))


def test_textbook_codewords():
    for m_txt, word in GOLD["codewords"].items():
        m = int(m_txt)
        for sign in (1, -1):
            c = sign * (m - 1)
            off, words = O.elias_encode(64, 127, 1, _codes(127, [c]))
            want = word + ("" if c == 0 else ("1" if c < 0 else "0"))
            got = _bits(words, int(off[1]))
            assert got[:len(want)] == want, (m, c)
            assert set(got[len(want):]) <= {"0"}          # pad bits are 0
            assert int(off[1]) == (len(want) + 31) // 32


def test_worked_stream():
    ws = GOLD["worked_stream"]
    n = len(ws["codes"])
    off, words = O.elias_encode(64, ws["s"], n, _codes(ws["s"], ws["codes"]))
    got = _bits(words, int(off[1]))
    assert got[:len(ws["bits"])] == ws["bits"]
    assert not int(got[len(ws["bits"]):] or "0", 2)


CASES = [(64, 1, 64 * 5 + 7), (128, 2, 128 * 3 + 1), (512, 4, 512 * 4 + 300),
         (512, 7, 512 * 2), (256, 127, 256 * 3 + 129), (1024, 3, 1024 * 2 + 65)]


def _random_codes(s, n, seed):
    """Codes with every magnitude present, most of them small."""
    rng = np.random.default_rng(seed)
    mag = np.minimum(rng.geometric(0.45, n) - 1, s)
    mag[rng.integers(0, n, 8)] = s
    return np.where(rng.random(n) < 0.5, -mag, mag)


@pytest.mark.parametrize("d,s,n", CASES)
def test_parser_and_lengths(d, s, n):
    vals = _random_codes(s, n, seed=d + s)
    off, words = O.elias_encode(d, s, n, _codes(s, vals))
    nb = (n + d - 1) // d
    assert off.size == nb + 1 and off[0] == 0
    for j in range(nb):
        blk = vals[j * d:(j + 1) * d]
        nbits = sum(2 * (abs(int(c)) + 1).bit_length() - 1 + (c != 0) for c in blk)
        nw = int(off[j + 1] - off[j])
        assert nw == (nbits + 31) // 32
        rec = _bits(words[int(off[j]):], nw)
        got, used = _parse(rec, blk.size)
        assert got == blk.tolist()
        assert used == nbits and not int(rec[used:] or "0", 2)


@pytest.mark.parametrize("d,s,n", CASES)
def test_round_trip(d, s, n):
    vals = _random_codes(s, n, seed=7 * d + s)
    codes = _codes(s, vals)
    off, words = O.elias_encode(d, s, n, codes)
    assert np.array_equal(O.elias_decode(d, s, n, off, words), codes)


@pytest.mark.parametrize("s,kind", [(1, "normal"), (4, "normal"), (4, "laplace"),
                                    (127, "heavy")])
def test_quantized_gradients_and_the_shannon_bound(s, kind):
    d = 512
    n = 512 * 40 + 77
    g = WL.small_mixture(n, seed=s, kind=kind)
    desc = O.Desc(O.UNIFORM, d, s=s)
    codes, _, _, _ = O.quantize(desc, g, seed=3, step=1)
    off, words = O.elias_encode(d, s, n, codes)
    assert np.array_equal(O.elias_decode(d, s, n, off, words), codes)
    vals = O.signed_codes(desc, n, codes)
    _, counts = np.unique(vals, return_counts=True)
    p = counts / n
    entropy = float(-(p * np.log2(p)).sum())
    # payload bits without the word padding of the records
    nbits = sum(2 * (abs(int(c)) + 1).bit_length() - 1 + (c != 0) for c in vals)
    assert nbits / n >= entropy - 1e-12
    assert 32 * int(off[-1]) >= nbits


@pytest.mark.parametrize("d,s,n", [(64, 1, 64 * 3 + 5), (512, 4, 1030), (128, 127, 300)])
def test_worst_case_size_and_all_zero(d, s, n):
    worst = np.array([s, -s] * n)[:n]
    off, _ = O.elias_encode(d, s, n, _codes(s, worst))
    assert int(off[-1]) == O.elias_max_words(d, s, n)
    off0, w0 = O.elias_encode(d, s, n, _codes(s, np.zeros(n, np.int64)))
    nb = (n + d - 1) // d
    assert np.array_equal(np.diff(off0),
                          [(min(d, n - j * d) + 31) // 32 for j in range(nb)])
    assert set(_bits(w0, int(off0[-1]))) <= {"0", "1"}
    assert all(_bits(w0[int(off0[j]):], 1)[0] == "1" for j in range(nb))


def test_rejections():
    with pytest.raises(ValueError):        # |c| = 4 > s = 2 in a 3-bit field
        O.elias_encode(64, 2, 4, _codes(2, [0, 1, -4, 2]))
    off, words = O.elias_encode(64, 4, 3, _codes(4, [1, 2, 3]))
    bad = words.copy()
    bad[0] = 0                                 # a run of zeros with no end
    with pytest.raises(ValueError):
        O.elias_decode(64, 4, 3, off, bad)
    with pytest.raises(ValueError):            # |c| + 1 = 9 > s + 1
        O.elias_decode(64, 4, 1, np.array([0, 1], np.uint64),
                       np.array([int("1001000", 2) << 0], np.uint32))
    with pytest.raises(ValueError):
        O.elias_encode(63, 4, 10, _codes(4, [0] * 10))
