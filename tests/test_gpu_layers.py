"""GPU parity of the per-layer scale (TernGrad layout, gq_quantize_layers /
gq_dequantize_accumulate_layers) against the oracle: layouts with empty,
one-element, tile-crossing and tile-sized layers, a tile met by more layers
than the kernels keep in LDS, every code width, dense packing, nearest
rounding, error feedback, aggregation of several payloads, the reduction to
the bucketed entry point when layers are cut at multiples of d, and the
160-layer 25.6M ternary gradient whole.  Codes, scales and residuals are
compared bit for bit."""
import numpy as np
import pytest

import oracle as O
from communication_efficient_gradient_amd import workloads as WL
from tests.parity import compare_codes, compare_values, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from communication_efficient_gradient_amd import gq
    return gq, torch


def _layout(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


LAYOUTS = {
    "mixed": [0, 1, 3, 2048, 0, 2047, 5000, 1, 1, 700, 0],
    "one_layer": [10_007],
    "tiny_many": [1] * 40 + [3] * 30 + [1000],   # > 32 layer starts in a tile
    "tile_sized": [2048] * 4 + [2049, 2047],
    "ragged": [5, 4099, 17, 65, 3000, 1],
    # layers spanning several 2048-element tiles, and 65 layer starts
    # within 5,240 elements
    "multi_tile": [4096] * 3 + [4097, 4095, 8192, 8191, 1],
    "many_starts": [100] * 45 + [37] * 20 + [9000],
    # 1024 layers or more: the layer search runs in global memory
    "over_1024_layers": [200] * 1100 + [7],
    "over_1024_tiny": [3] * 1200 + [5000],
}


def run_layers(dev, desc, off, g, e, seed, step):
    gq, torch = dev
    gd = gq.desc(desc.scheme, desc.d, desc.s, desc.L, desc.flags, desc.clip_sigma)
    n = g.size
    nl = off.size - 1
    G = torch.from_numpy(g).cuda()
    E = None if e is None else torch.from_numpy(e.copy()).cuda()
    OFF = torch.from_numpy(off).cuda()
    _, cap, _ = gq.gq_payload_size(gd, n)
    codes = torch.full((cap,), 0xAB, dtype=torch.uint8, device="cuda")
    meta = torch.full((nl,), float("nan"), device="cuda")
    gq.gq_quantize_layers(gd, OFF, G, E, seed, step, codes, meta)
    torch.cuda.synchronize()
    return gd, OFF, codes, meta, E


def check_layers(dev, desc, sizes, seed=1, step=0, ef=True):
    gq, torch = dev
    off = _layout(sizes)
    n = int(off[-1])
    say(f"layers s={desc.s} flags={desc.flags} n={n} nl={off.size - 1} ef={ef}")
    g = WL.small_mixture(n, seed=n + desc.s, kind="laplace")
    e = (WL.small_mixture(n, seed=n + 1) * np.float32(0.1)) if ef else None
    rc, rm, re_ = O.quantize_layers(desc, off, g, e, seed=seed, step=step)
    gd, OFF, codes, meta, E = run_layers(dev, desc, off, g, e, seed, step)
    compare_codes(desc, n, codes.cpu().numpy(), rc)
    assert np.array_equal(meta.cpu().numpy(), rm)
    if ef:
        assert np.array_equal(E.cpu().numpy().view(np.uint32), re_.view(np.uint32))
    out = torch.full((n,), float("nan"), device="cuda")
    gq.gq_dequantize_accumulate_layers(gd, n, OFF, [codes], [meta], 1.0, 0.0, out)
    torch.cuda.synchronize()
    xr = O.dequantize_accumulate_layers(desc, off, n, [rc], [rm])
    assert np.array_equal(out.cpu().numpy().view(np.uint32), xr.view(np.uint32))


@pytest.mark.parametrize("name", sorted(LAYOUTS))
@pytest.mark.parametrize("s", [1, 4, 127])
def test_layouts(dev, name, s):
    check_layers(dev, O.Desc(O.UNIFORM, s=s), LAYOUTS[name], seed=s, step=2)


@pytest.mark.parametrize("name", ["mixed", "tiny_many", "ragged"])
@pytest.mark.parametrize("s,flags", [(1, O.FLAG_DENSE), (3, O.FLAG_DENSE),
                                     (1, O.FLAG_NEAREST), (7, O.FLAG_DENSE | O.FLAG_NEAREST),
                                     (2, 0)])
def test_dense_and_nearest(dev, name, s, flags):
    check_layers(dev, O.Desc(O.UNIFORM, s=s, flags=flags), LAYOUTS[name], seed=5)


def test_no_error_feedback(dev):
    check_layers(dev, O.Desc(O.UNIFORM, s=1), LAYOUTS["mixed"], ef=False)


@pytest.mark.parametrize("W", [2, 3, 8])
def test_aggregate(dev, W):
    gq, torch = dev
    desc = O.Desc(O.UNIFORM, s=127)
    off = _layout(LAYOUTS["mixed"])
    n = int(off[-1])
    cl, ml = [], []
    for w in range(W):
        g = WL.small_mixture(n, seed=300 + w)
        c, m, _ = O.quantize_layers(desc, off, g, seed=w)
        cl.append(c)
        ml.append(m)
    gd = gq.desc(0, 512, s=127)
    OFF = torch.from_numpy(off).cuda()
    C = [torch.from_numpy(np.concatenate([c, np.zeros(16, np.uint8)])).cuda() for c in cl]
    M = [torch.from_numpy(m).cuda() for m in ml]
    out0 = WL.small_mixture(n, seed=7)
    out = torch.from_numpy(out0.copy()).cuda()
    gq.gq_dequantize_accumulate_layers(gd, n, OFF, C, M, 1.0 / W, 0.5, out)
    torch.cuda.synchronize()
    ref = O.dequantize_accumulate_layers(desc, off, n, cl, ml, 1.0 / W, 0.5, out0)
    layer = np.repeat(np.arange(off.size - 1), np.diff(off))
    scale = np.abs(0.5 * out0.astype(np.float64))
    for c, m in zip(cl, ml):
        k = O.signed_codes(desc, n, c).astype(np.float64)
        scale += np.abs(k * (m[layer] / 127.0)) / W
    compare_values(out.cpu().numpy(), ref, scale)


def test_equal_chunks_match_the_bucketed_entry_point(dev):
    gq, torch = dev
    n, d = 9 * 512 + 77, 512
    g = WL.small_mixture(n, seed=11, kind="laplace")
    off = np.array(list(range(0, n, d)) + [n], dtype=np.int64)
    desc = O.Desc(O.UNIFORM, d, s=1)
    gd, OFF, codes, meta, E = run_layers(dev, desc, off, g, np.zeros(n, np.float32), 4, 1)
    G = torch.from_numpy(g).cuda()
    E2 = torch.zeros(n, device="cuda")
    c2, m2 = gq.alloc_payload(gd, n)
    gq.gq_quantize(gd, G, E2, 4, 1, c2, m2)
    torch.cuda.synchronize()
    cb = desc.code_bytes(n)
    assert torch.equal(codes[:cb], c2[:cb])
    assert torch.equal(meta.view(torch.int32), m2.view(torch.int32))
    assert torch.equal(E.view(torch.int32), E2.view(torch.int32))


def test_ternary_160_layers_whole(dev):
    """The 25.6M-element ternary gradient with one scale per layer (its 160
    Laplace layers), two error-feedback steps, everything bit for bit."""
    gq, torch = dev
    sizes, _ = WL.ternary_layout()
    off = _layout(sizes)
    n = int(off[-1])
    desc = O.Desc(O.UNIFORM, s=1)
    gd = gq.desc(0, 512, s=1)
    OFF = torch.from_numpy(off).cuda()
    E = torch.zeros(n, device="cuda")
    e_ref = np.zeros(n, np.float32)
    _, cap, _ = gq.gq_payload_size(gd, n)
    codes = torch.empty(cap, dtype=torch.uint8, device="cuda")
    meta = torch.empty(off.size - 1, device="cuda")
    out = torch.empty(n, device="cuda")
    for t in range(2):
        say(f"ternary layers step {t}")
        g = WL.ternary_gradient(t)
        gq.gq_quantize_layers(gd, OFF, torch.from_numpy(g).cuda(), E, 2, t, codes, meta)
        gq.gq_dequantize_accumulate_layers(gd, n, OFF, [codes], [meta], 1.0, 0.0, out)
        torch.cuda.synchronize()
        rc, rm, e_ref = O.quantize_layers(desc, off, g, e_ref, seed=2, step=t)
        compare_codes(desc, n, codes.cpu().numpy(), rc)
        assert np.array_equal(meta.cpu().numpy(), rm)
        assert np.array_equal(E.cpu().numpy().view(np.uint32), e_ref.view(np.uint32))
        xr = O.dequantize_accumulate_layers(desc, off, n, [rc], [rm])
        assert np.array_equal(out.cpu().numpy().view(np.uint32), xr.view(np.uint32))
