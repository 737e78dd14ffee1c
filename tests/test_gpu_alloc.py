"""GPU parity of gq_allocate_layer_bits (layer-wise bit allocation) against
the oracle's allocate_layer_bits and alloc_segments: widths and segment
offsets bit for bit over layouts from 1 to 1024 layers, with empty layers,
zero scales, exactly equal scales (ties broken by layer, then width) and
budgets from 2 to 8 bits per element and beyond; argument errors before any
launch."""
import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from communication_efficient_gradient_amd import gq
    return gq, torch


def run(dev, sizes, scales, budget):
    gq, torch = dev
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    nl = len(sizes)
    OFF = torch.from_numpy(off).cuda()
    S = torch.from_numpy(np.asarray(scales, dtype=np.float32)).cuda()
    Wd = torch.full((nl,), -1, dtype=torch.int32, device="cuda")
    Sg = torch.full((nl + 1,), -1, dtype=torch.int64, device="cuda")
    gq.gq_allocate_layer_bits(n, OFF, S, budget, Wd, Sg)
    torch.cuda.synchronize()
    return Wd.cpu().numpy().tolist(), Sg.cpu().numpy().tolist()


@pytest.mark.parametrize("nl", [1, 7, 160, 1000, 1024])
@pytest.mark.parametrize("seed", range(4))
def test_widths_and_segments_match_the_oracle(dev, nl, seed):
    rng = np.random.default_rng(1000 * nl + seed)
    sizes = rng.integers(0, 3000, nl)
    sizes[rng.random(nl) < 0.05] = 0
    pool = np.float32(np.exp(rng.uniform(-9, -3, max(1, nl // 3))))
    scales = rng.choice(pool, nl).astype(np.float32)  # repeated values: ties
    scales[rng.random(nl) < 0.05] = 0.0
    n = int(sizes.sum())
    if n == 0:
        sizes[0] = 1
        n = 1
    for budget in (2 * n, int(rng.integers(2 * n, 8 * n + 1)), 4 * n, 8 * n, 9 * n):
        ref_w, _ = O.allocate_layer_bits(sizes.tolist(), scales.tolist(), budget)
        ref_s = O.alloc_segments(sizes.tolist(), ref_w)
        got_w, got_s = run(dev, sizes.tolist(), scales.tolist(), budget)
        assert got_w == ref_w, (nl, seed, budget)
        assert got_s == ref_s, (nl, seed, budget)


def test_the_160_layer_gradient(dev):
    """The layered 25.6M gradient's layout and per-layer max-abs scales from
    gq_quantize_layers, at 3 bits per element."""
    gq, torch = dev
    from communication_efficient_gradient_amd import workloads as WL
    sizes, _ = WL.ternary_layout()
    g = WL.ternary_gradient(0)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    d = gq.desc(0, 512, s=1)
    codes, _ = gq.alloc_payload(d, g.size)
    meta = torch.empty(len(sizes), device="cuda")
    gq.gq_quantize_layers(d, torch.from_numpy(off).cuda(), torch.from_numpy(g).cuda(),
                          None, 1, 0, codes, meta)
    torch.cuda.synchronize()
    scales = meta.cpu().numpy()
    budget = 3 * g.size
    ref_w, _ = O.allocate_layer_bits([int(x) for x in sizes], scales.tolist(), budget)
    got_w, got_s = run(dev, [int(x) for x in sizes], scales, budget)
    assert got_w == ref_w
    assert got_s == O.alloc_segments([int(x) for x in sizes], ref_w)
    assert len(set(ref_w)) > 1  # the budget spreads widths over the layers


def test_argument_errors(dev):
    gq, torch = dev
    off = torch.tensor([0, 10, 20], dtype=torch.int64, device="cuda")
    s = torch.ones(2, device="cuda")
    w = torch.empty(2, dtype=torch.int32, device="cuda")
    sg = torch.empty(3, dtype=torch.int64, device="cuda")
    with pytest.raises(gq.GQError) as ei:
        gq.gq_allocate_layer_bits(20, off, s, 39, w, sg)  # below 2 bits each
    assert ei.value.status == gq.GQ_EINVAL
    big = torch.zeros(1026, dtype=torch.int64, device="cuda")
    s2 = torch.ones(1025, device="cuda")
    w2 = torch.empty(1025, dtype=torch.int32, device="cuda")
    sg2 = torch.empty(1026, dtype=torch.int64, device="cuda")
    with pytest.raises(gq.GQError) as ei:
        gq.gq_allocate_layer_bits(1, big, s2, 100, w2, sg2)
    assert ei.value.status == gq.GQ_EUNSUPPORTED
