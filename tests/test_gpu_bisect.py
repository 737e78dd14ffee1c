"""GPU parity of ORQ levels by recursive bisection (GQ_FLAG_BISECT, d <=
512) against the oracle: every bucket size of the lane-group kernel, L from
3 to 16 (full rounds and rounds that keep their largest gains), clipping,
dense packing, nearest rounding, error feedback, a skewed bucket where
bisection and the greedy differ, and buckets of small integers whose gains
tie exactly.  The 100M ORQ-5 / ORQ-9 gradients are compared whole in
test_gpu_full.py."""
import numpy as np
import pytest

import oracle as O
from communication_efficient_gradient_amd import workloads as WL
from tests.parity import say
from tests.test_gpu_small import check_quantize, dev, run_gpu  # noqa: F401

pytestmark = pytest.mark.gpu

B = O.FLAG_BISECT


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("L", [3, 5, 6, 9, 12, 16])
@pytest.mark.parametrize("clip", [0, O.FLAG_CLIP])
def test_bisect_every_bucket(dev, d, L, clip):
    n = 3 * d + 45
    g = WL.orq_gradient(n)
    check_quantize(dev, O.Desc(O.ORQ, d, L=L, flags=B | clip, clip_sigma=3.0),
                   g, None, seed=L)


@pytest.mark.parametrize("flags", [B | O.FLAG_DENSE, B | O.FLAG_NEAREST,
                                   B | O.FLAG_DENSE | O.FLAG_NEAREST])
def test_bisect_with_other_flags(dev, flags):
    n = 4 * 512 + 7
    g = WL.small_mixture(n, seed=flags, kind="heavy")
    e = WL.small_mixture(n, seed=flags + 1) * np.float32(0.05)
    for L in (5, 9):
        check_quantize(dev, O.Desc(O.ORQ, 512, L=L, flags=flags), g, e, seed=2, step=3)


def test_skewed_buckets_where_the_readings_differ(dev):
    rng = np.random.default_rng(1)
    blocks = []
    for k in range(8):
        blocks.append(np.concatenate([rng.uniform(0, 1, 480),
                                      rng.uniform(-10, 0, 32)]))
    g = np.concatenate(blocks).astype(np.float32)
    desc = O.Desc(O.ORQ, 512, L=5, flags=B)
    _, mb, _, _ = O.quantize(desc, g)
    _, mg, _, _ = O.quantize(O.Desc(O.ORQ, 512, L=5), g)
    assert not np.array_equal(mb, mg)
    check_quantize(dev, desc, g, None, seed=4)


def test_exact_tie_rounds_bit_for_bit(dev):
    """Buckets of small integers, where gains tie exactly in any fp64 order:
    the kernel's partial rounds take the smaller value on equal gains like
    the oracle, so levels and codes must agree in every bucket, flagged ties
    included."""
    gq, torch = dev
    from tests.test_gpu_small import run_gpu
    rows = [np.array([-6, -6, -4, -2, -1, -1, -1, -1, 0, 0, 1, 2, 6, 6, 6, 6, 6]
                     + [6] * 47, dtype=np.float32)]
    for s in range(63):
        rng = np.random.default_rng(7000 + s)
        rows.append(rng.integers(-6, 7, 64).astype(np.float32))
    g = np.concatenate(rows)
    for L in (7, 8, 9):
        d = O.Desc(O.ORQ, 64, L=L, flags=B)
        say(f"bisect exact ties L={L} n={g.size}")
        rc, rm, _, tie = O.quantize(d, g, None, seed=5, step=0)
        gc, gm, _ = run_gpu(dev, d, g, None, 5, 0)
        assert tie.sum() > 0
        assert np.array_equal(gm, rm)
        assert np.array_equal(gc[:d.code_bytes(g.size)], rc)
