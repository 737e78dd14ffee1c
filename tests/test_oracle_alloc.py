"""Pins of the oracle's layer-wise bit allocation ("Gradient Quantization"
glossary, layer-wise quantization paragraph: wider codes for layers with
larger gradient variance) and of its mixed-width payload.

The allocation is pinned to what holds for any correct greedy on convex
per-layer costs: brute force over every allocation of small layouts (no
allocation using at most as many bits has a smaller variance bound, computed
in exact rationals), monotonicity of the widths in the layer scale, the
budget and its extremes.  The payload is pinned to properties of the
rounding: every decoded value lies on its layer's grid next to p, error
feedback keeps p - x_hat exactly, segments have the stated sizes with zero
padding, and aggregation matches exact rational sums."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

WIDTHS = O.ALLOC_WIDTHS


def bound(sizes, scales, widths):
    """Sum over layers of n_l * M_l^2 / (4 s_l^2), exactly."""
    tot = Fraction(0)
    for n_l, m, b in zip(sizes, scales, widths):
        s = (1 << (b - 1)) - 1
        tot += Fraction(int(n_l)) * Fraction(float(np.float32(m))) ** 2 / (4 * s * s)
    return tot


def bits(sizes, widths):
    return sum(int(n) * b for n, b in zip(sizes, widths))


def random_layout(rng, nl):
    sizes = rng.integers(0, 41, nl)
    scales = rng.choice([0.0, 1e-3, 2e-3, 0.5e-3, 3e-3], nl) * rng.choice([1.0, 1.5], nl)
    return [int(x) for x in sizes], [float(np.float32(x)) for x in scales]


@pytest.mark.parametrize("seed", range(120))
def test_no_allocation_with_fewer_bits_has_a_smaller_bound(seed):
    rng = np.random.default_rng(seed)
    nl = int(rng.integers(1, 6))
    sizes, scales = random_layout(rng, nl)
    n = sum(sizes)
    budget = int(rng.integers(2 * n, 8 * n + 11))
    widths, used = O.allocate_layer_bits(sizes, scales, budget)
    assert used == bits(sizes, widths) <= budget
    best = min(bound(sizes, scales, w) for w in itertools.product(WIDTHS, repeat=nl)
               if bits(sizes, w) <= used)
    assert bound(sizes, scales, widths) == best


def test_widths_grow_with_the_layer_scale():
    rng = np.random.default_rng(7)
    for _ in range(30):
        nl = 24
        sizes = [int(x) for x in rng.integers(1, 5000, nl)]
        scales = [float(np.float32(x)) for x in np.exp(rng.uniform(-9, -3, nl))]
        n = sum(sizes)
        widths, _ = O.allocate_layer_bits(sizes, scales, int(rng.integers(2 * n, 8 * n)))
        for a in range(nl):
            for b in range(nl):
                if scales[a] > scales[b]:
                    assert widths[a] >= widths[b]


def test_budget_extremes_and_zero_layers():
    sizes = [10, 0, 30, 5]
    scales = [1e-3, 2e-3, 0.0, 4e-3]
    w, used = O.allocate_layer_bits(sizes, scales, 2 * sum(sizes))
    assert w == [2, 2, 2, 2] and used == 2 * sum(sizes)
    w, used = O.allocate_layer_bits(sizes, scales, 8 * sum(sizes))
    # every layer that has elements and a nonzero scale reaches 8 bits; the
    # all-zero layer gains nothing and keeps 2, the empty one costs nothing
    assert w == [8, 2, 2, 8]
    with pytest.raises(ValueError):
        O.allocate_layer_bits(sizes, scales, 2 * sum(sizes) - 1)


def test_larger_budgets_never_raise_the_bound():
    rng = np.random.default_rng(3)
    sizes, scales = random_layout(rng, 12)
    n = sum(sizes)
    prev = None
    for budget in range(2 * n, 8 * n + 1, max(1, n // 7)):
        w, _ = O.allocate_layer_bits(sizes, scales, budget)
        cur = bound(sizes, scales, w)
        assert prev is None or cur <= prev
        prev = cur


def _layout():
    sizes = np.array([0, 1, 37, 512, 1000, 3, 0, 777, 64, 2049])
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64), sizes


def test_payload_values_on_each_layers_grid_with_exact_residual():
    off, sizes = _layout()
    n = int(off[-1])
    rng = np.random.default_rng(11)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    e = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    widths = [int(x) for x in rng.choice(WIDTHS, sizes.size)]
    pay, meta, e_new = O.quantize_layers_alloc(off, g, e, widths, seed=5, step=2)
    seg = O.alloc_segments(sizes, widths)
    assert pay.size == seg[-1]
    x = O.dequantize_layers_alloc(off, n, pay, meta, widths)
    p = (g + e).astype(np.float32)
    for lay, b in enumerate(widths):
        lo, hi = int(off[lay]), int(off[lay + 1])
        nbytes = (int(sizes[lay]) * b + 7) // 8
        assert seg[lay + 1] - seg[lay] == (nbytes + 15) // 16 * 16
        assert not pay[seg[lay] + nbytes:seg[lay + 1]].any()  # zero padding
        if hi == lo:
            continue
        s = (1 << (b - 1)) - 1
        assert meta[lay] == np.max(np.abs(p[lo:hi]))
        step = np.float64(np.float32(meta[lay] / np.float32(s)))
        k = np.rint(x[lo:hi] / step) if step > 0 else np.zeros(hi - lo)
        assert np.all(np.abs(k) <= s)
        assert np.all(np.abs(x[lo:hi] - k * step) <= 1e-6 * np.abs(x[lo:hi]) + 1e-30)
        assert np.all(np.abs(p[lo:hi].astype(np.float64) - x[lo:hi]) <= step * (1 + 1e-6))
    assert np.array_equal(e_new.view(np.uint32), (p - x).astype(np.float32).view(np.uint32))


def test_one_width_everywhere_is_the_per_layer_path():
    off, sizes = _layout()
    n = int(off[-1])
    g = (np.random.default_rng(2).standard_normal(n) * 1e-3).astype(np.float32)
    for b in WIDTHS:
        pay, meta, _ = O.quantize_layers_alloc(off, g, None, [b] * sizes.size, seed=3)
        d = O.Desc(O.UNIFORM, 512, s=(1 << (b - 1)) - 1)
        codes, m, _ = O.quantize_layers(d, off, g, None, seed=3)
        assert np.array_equal(meta, m)
        ref = O.dequantize_accumulate_layers(d, off, n, [codes], [m])
        got = O.dequantize_layers_alloc(off, n, pay, meta, [b] * sizes.size)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_aggregate_is_the_exact_sum_rounded_once():
    off, sizes = _layout()
    n = int(off[-1])
    rng = np.random.default_rng(9)
    pays, metas, wl, xs = [], [], [], []
    for w in range(3):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        widths = [int(x) for x in rng.choice(WIDTHS, sizes.size)]
        pay, meta, _ = O.quantize_layers_alloc(off, g, None, widths, seed=w)
        pays.append(pay)
        metas.append(meta)
        wl.append(widths)
        xs.append(O.dequantize_layers_alloc(off, n, pay, meta, widths))
    out0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    got = O.dequantize_accumulate_layers_alloc(off, n, pays, metas, wl, 1 / 3, 0.5, out0)
    for i in range(0, n, 97):
        exact = Fraction(0.5) * Fraction(float(out0[i])) + Fraction(1 / 3) * sum(
            Fraction(float(x[i])) for x in xs)
        ref = np.float32(float(exact))
        assert abs(float(got[i]) - float(ref)) <= 1e-6 * (abs(float(ref)) + 1e-30)


def test_gain_is_per_added_bit():
    """Hand-worked: two layers of 10 elements, M = 3e-3 and 1e-3.  Bound
    reductions per added bit, M^2 (1/s^2 - 1/s'^2) / (4 (b' - b)):
    A 2->3 2.0e-6, B 2->3 2.2e-7, A 3->4 2.0e-7, B 3->4 2.3e-8, A 4->8
    1.1e-8 (a 4->8 step adds 4 bits per element).  With 100 bits: A, B to 3
    (60 bits), A, B to 4 (80 bits), then A 4->8 needs 40 more: stop at
    (4, 4).  Ranking the 4->8 step by its whole reduction (4.6e-8, above
    B 3->4) would stop at (4, 3) with 70 bits."""
    widths, used = O.allocate_layer_bits([10, 10], [3e-3, 1e-3], 100)
    assert widths == [4, 4] and used == 80
    widths, used = O.allocate_layer_bits([10, 10], [3e-3, 1e-3], 120)
    assert widths == [8, 4] and used == 120
