"""Host model of how the allocation-payload quantizer divides its work: one
thread per 32-bit payload word, at 3 bits one thread per three words of a
segment (32 whole codes).  Checked over random layouts and width mixes:

- every element of the gradient is coded by exactly one thread;
- every word of every segment is written by exactly one thread, and no
  word past the last segment;
- the element runs of the threads of one 64-lane wave are consecutive and
  span at most 1024 elements (the wave's LDS row);
- the words the threads assemble from their codes are the oracle's packing
  of each layer (LSB-first, segments padded to 16 bytes), and the reads of
  the dequantizer (one word, or two when a 3-bit code straddles) stay
  inside the segments.

This is a design aid for the kernel's indexing, written in Python: it can
pass while the HIP code drifts from it.  The kernel itself is checked by
tests/test_gpu_alloc_payload.py, whose payloads, maxima and residuals must
equal the oracle's bit for bit, with the bytes past the last segment
checked untouched."""
import numpy as np
import pytest

import oracle as O

WAVE_ELEMS = 1024


def layer_of(off, nl, x):
    lo, hi = 0, nl
    while hi - lo > 1:
        mid = (lo + hi) >> 1
        if off[mid] <= x:
            lo = mid
        else:
            hi = mid
    return lo


def thread_runs(sizes, widths):
    """(word, layer, width, first element, end element, words written) of
    every thread that codes, as the kernel assigns them."""
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n, nl = int(off[-1]), len(sizes)
    seg = O.alloc_segments(sizes, widths)
    cap_words = (n + 16 * nl) // 4
    out = []
    for w in range(cap_words):
        if 4 * w >= seg[nl]:
            break
        lay = layer_of(seg, nl, 4 * w)
        b = widths[lay]
        nw = 3 if b == 3 else 1
        sw0, sw1 = seg[lay] // 4, seg[lay + 1] // 4
        if (w - sw0) % nw:
            continue
        lo, nlay = int(off[lay]), int(off[lay + 1] - off[lay])
        assert (32 * (w - sw0)) % b == 0
        kfirst = 32 * (w - sw0) // b
        kend = max(kfirst, min(kfirst + 32 * nw // b, nlay))
        words = [w + m for m in range(nw) if m == 0 or (w + m < sw1 and w + m < cap_words)]
        out.append((w, lay, b, lo + kfirst, lo + kend, words))
    return off, seg, out


LAYOUT_SIZES = [0, 1, 2, 3, 5, 17, 31, 32, 33, 63, 64, 65, 95, 96, 97, 100,
                500, 1023, 1024, 1025, 3000]


@pytest.mark.parametrize("seed", range(40))
def test_work_division(seed):
    rng = np.random.default_rng(seed)
    nl = int(rng.integers(1, 30))
    sizes = [int(x) for x in rng.choice(LAYOUT_SIZES, nl)]
    if sum(sizes) == 0:
        sizes[0] = 7
    widths = [int(x) for x in rng.choice(O.ALLOC_WIDTHS, nl)]
    off, seg, runs = thread_runs(sizes, widths)
    n = int(off[-1])
    coded = np.zeros(n, dtype=np.int64)
    written = np.zeros(seg[-1] // 4, dtype=np.int64)
    for _, _, _, i0, i1, words in runs:
        coded[i0:i1] += 1
        for w in words:
            assert w < seg[-1] // 4
            written[w] += 1
    assert np.all(coded == 1)
    assert np.all(written == 1)
    # per wave: consecutive runs within one LDS row
    waves = {}
    for w, _, _, i0, i1, _ in runs:
        if i1 > i0:
            waves.setdefault(w // 64, []).append((i0, i1))
    for rs in waves.values():
        for (_, a1), (b0, _) in zip(rs, rs[1:]):
            assert a1 == b0
        assert rs[-1][1] - rs[0][0] <= WAVE_ELEMS


@pytest.mark.parametrize("seed", range(10))
def test_assembled_words_are_the_oracle_packing(seed):
    rng = np.random.default_rng(100 + seed)
    nl = int(rng.integers(1, 12))
    sizes = [int(x) for x in rng.choice(LAYOUT_SIZES, nl)]
    if sum(sizes) == 0:
        sizes[0] = 9
    widths = [int(x) for x in rng.choice(O.ALLOC_WIDTHS, nl)]
    off, seg, runs = thread_runs(sizes, widths)
    n = int(off[-1])
    fields = np.zeros(n, dtype=np.uint32)
    for lay in range(nl):
        lo, hi = int(off[lay]), int(off[lay + 1])
        fields[lo:hi] = rng.integers(0, 1 << widths[lay], hi - lo)
    words = np.zeros(seg[-1] // 4, dtype=np.uint64)
    for _, _, b, i0, i1, ws in runs:
        acc = 0
        for j, i in enumerate(range(i0, i1)):
            acc |= int(fields[i]) << (j * b)
        for m, w in enumerate(ws):
            words[w] = (acc >> (32 * m)) & 0xFFFFFFFF
    got = words.astype(np.uint32).view(np.uint8)
    ref = np.zeros(seg[-1], dtype=np.uint8)
    for lay in range(nl):
        lo, hi = int(off[lay]), int(off[lay + 1])
        if hi > lo:
            packed = O.pack(widths[lay], fields[lo:hi])
            ref[seg[lay]:seg[lay] + packed.size] = packed
    assert np.array_equal(got, ref)
    # the dequantizer's reads
    u32 = got.view(np.uint32)
    for i in range(n):
        lay = layer_of(off, nl, i)
        b = widths[lay]
        bit = 8 * seg[lay] + (i - int(off[lay])) * b
        wi, sh = bit >> 5, bit & 31
        assert 8 * seg[lay] <= 32 * wi and wi < seg[lay + 1] // 4
        v = int(u32[wi]) >> sh
        if sh + b > 32:
            assert wi + 1 < seg[lay + 1] // 4
            v |= int(u32[wi + 1]) << (32 - sh)
        assert v & ((1 << b) - 1) == fields[i]
