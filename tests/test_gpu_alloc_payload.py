"""GPU parity of the layer-wise allocation payload: gq_quantize_layers_alloc
against the oracle's quantize_layers_alloc (payload bytes, layer maxima and
residuals bit for bit; bytes past the last segment untouched) and
gq_dequantize_accumulate_layers_alloc against
dequantize_accumulate_layers_alloc (the stated value tolerance), over
layouts with empty, one-element and ragged layers, every width and width
mix, random rounding and rounding to the nearest level, and widths and
segments taken straight from gq_allocate_layer_bits on the device."""
import numpy as np
import pytest

import oracle as O
from communication_efficient_gradient_amd import workloads as WL
from tests.parity import compare_values, say

pytestmark = pytest.mark.gpu

WIDTHS = list(O.ALLOC_WIDTHS)
FILL = 0xAB


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
    "tiny_many": [1] * 40 + [3] * 30 + [1000],
    "ragged": [5, 4099, 17, 65, 3000, 1, 31, 33, 95, 97],
    "over_1024_layers": [50] * 1100 + [7],
}


def quantize_gpu(dev, off, g, e, widths, seed, step, flags=0):
    gq, torch = dev
    n, nl = g.size, off.size - 1
    sizes = np.diff(off)
    seg = np.asarray(O.alloc_segments(sizes, widths), dtype=np.int64)
    cap = gq.gq_alloc_payload_bytes(n, nl)
    OFF = torch.from_numpy(off).cuda()
    Wd = torch.from_numpy(np.asarray(widths, dtype=np.int32)).cuda()
    Sg = torch.from_numpy(seg).cuda()
    P = torch.full((cap,), FILL, dtype=torch.uint8, device="cuda")
    M = torch.full((nl,), -1.0, dtype=torch.float32, device="cuda")
    G = torch.from_numpy(g).cuda()
    E = None if e is None else torch.from_numpy(e.copy()).cuda()
    gq.gq_quantize_layers_alloc(OFF, G, E, Wd, Sg, seed, step, P, M, flags=flags)
    torch.cuda.synchronize()
    return (P.cpu().numpy(), M.cpu().numpy(),
            None if E is None else E.cpu().numpy(), seg)


def check_quantize(dev, sizes, widths, seed=1, step=0, ef=True, flags=0):
    off = _layout(sizes)
    n = int(off[-1])
    g = WL.small_mixture(n, seed=seed)
    e = WL.small_mixture(n, seed=seed + 50) * np.float32(0.05) if ef else None
    say(f"alloc quantize: n={n} nl={off.size - 1} widths={sorted(set(widths))} "
        f"seed={seed} ef={ef} flags={flags}")
    pay, meta, e_new, seg = quantize_gpu(dev, off, g, e, widths, seed, step, flags)
    rp, rm, re = O.quantize_layers_alloc(off, g, e, widths, seed=seed, step=step,
                                         flags=flags)
    total = int(seg[-1])
    assert rp.size == total
    assert np.array_equal(meta.view(np.uint32), rm.view(np.uint32))
    diff = np.nonzero(pay[:total] != rp)[0]
    assert diff.size == 0, f"{diff.size} payload bytes differ, first at {diff[:5]}"
    assert np.all(pay[total:] == FILL), "bytes past the last segment were written"
    if ef:
        assert np.array_equal(e_new.view(np.uint32), re.view(np.uint32))


@pytest.mark.parametrize("name", list(LAYOUTS))
@pytest.mark.parametrize("mix", ["random", 2, 3, 4, 8])
def test_payload_matches_the_oracle(dev, name, mix):
    sizes = LAYOUTS[name]
    rng = np.random.default_rng(len(sizes) * 31 + (0 if mix == "random" else mix))
    widths = ([int(x) for x in rng.choice(WIDTHS, len(sizes))] if mix == "random"
              else [mix] * len(sizes))
    check_quantize(dev, sizes, widths, seed=3, step=2)


@pytest.mark.parametrize("flags", [0, 4])
def test_without_error_feedback_and_nearest(dev, flags):
    sizes = LAYOUTS["ragged"]
    widths = [3, 2, 8, 4, 3, 3, 2, 3, 4, 8]
    check_quantize(dev, sizes, widths, seed=9, ef=False, flags=flags)
    check_quantize(dev, sizes, widths, seed=9, ef=True, flags=flags)


def test_zero_layers(dev):
    """All-zero layers: scale 0, every code 0 and the residual p itself."""
    gq, torch = dev
    sizes = [100, 333, 64]
    off = _layout(sizes)
    g = WL.small_mixture(int(off[-1]), seed=4)
    g[100:433] = 0.0
    widths = [3, 3, 8]
    pay, meta, _, seg = quantize_gpu(dev, off, g, None, widths, 0, 0)
    rp, rm, _ = O.quantize_layers_alloc(off, g, None, widths, seed=0, step=0)
    assert meta[1] == 0.0
    assert np.array_equal(pay[:seg[-1]], rp)
    assert not pay[seg[1]:seg[2]].any()


def test_allocation_then_quantize_on_the_device(dev):
    """The widths and segments gq_allocate_layer_bits writes feed the
    quantizer without a host round trip."""
    gq, torch = dev
    sizes = [3000, 17, 0, 4099, 700, 1, 2048, 5000]
    off = _layout(sizes)
    n = int(off[-1])
    nl = off.size - 1
    rng = np.random.default_rng(5)
    g = WL.small_mixture(n, seed=5)
    for lay in range(nl):  # layers of very different spread
        g[off[lay]:off[lay + 1]] *= np.float32(np.exp(rng.uniform(-4, 2)))
    OFF = torch.from_numpy(off).cuda()
    G = torch.from_numpy(g).cuda()
    M0 = torch.empty(nl, dtype=torch.float32, device="cuda")
    Wd = torch.empty(nl, dtype=torch.int32, device="cuda")
    Sg = torch.empty(nl + 1, dtype=torch.int64, device="cuda")
    cap = gq.gq_alloc_payload_bytes(n, nl)
    P = torch.full((cap,), FILL, dtype=torch.uint8, device="cuda")
    M = torch.empty(nl, dtype=torch.float32, device="cuda")
    gd = gq.desc(0, 512, s=1)
    codes0, _ = gq.alloc_payload(gd, n)
    for budget in (2 * n, 3 * n, 5 * n, 8 * n):
        gq.gq_quantize_layers(gd, OFF, G, None, 0, 0, codes0, M0)  # the scales
        gq.gq_allocate_layer_bits(n, OFF, M0, budget, Wd, Sg)
        gq.gq_quantize_layers_alloc(OFF, G, None, Wd, Sg, 7, 1, P, M)
        torch.cuda.synchronize()
        widths = Wd.cpu().numpy().tolist()
        ref_w, _ = O.allocate_layer_bits(sizes, M0.cpu().numpy().tolist(), budget)
        assert widths == ref_w
        rp, rm, _ = O.quantize_layers_alloc(off, g, None, widths, seed=7, step=1)
        got = P.cpu().numpy()
        assert np.array_equal(got[:rp.size], rp), budget
        assert np.array_equal(M.cpu().numpy(), rm)


def dequantize_case(dev, sizes, W, seed, alpha, beta):
    gq, torch = dev
    off = _layout(sizes)
    n, nl = int(off[-1]), off.size - 1
    rng = np.random.default_rng(seed)
    pays, metas, wl = [], [], []
    for w in range(W):
        g = WL.small_mixture(n, seed=seed * 100 + w)
        widths = [int(x) for x in rng.choice(WIDTHS, nl)]
        p, m, _ = O.quantize_layers_alloc(off, g, None, widths, seed=w)
        pays.append(p)
        metas.append(m)
        wl.append(widths)
    out0 = WL.small_mixture(n, seed=seed + 7)
    say(f"alloc dequantize: n={n} nl={nl} W={W} alpha={alpha} beta={beta}")
    OFF = torch.from_numpy(off).cuda()
    P = [torch.from_numpy(np.concatenate([p, np.zeros(16, np.uint8)])).cuda() for p in pays]
    M = [torch.from_numpy(m).cuda() for m in metas]
    Wd = [torch.from_numpy(np.asarray(w, dtype=np.int32)).cuda() for w in wl]
    Sg = [torch.from_numpy(np.asarray(O.alloc_segments(np.diff(off), w),
                                      dtype=np.int64)).cuda() for w in wl]
    out = torch.from_numpy(out0.copy()).cuda()
    gq.gq_dequantize_accumulate_layers_alloc(n, OFF, P, M, Wd, Sg, alpha, beta, out)
    torch.cuda.synchronize()
    ref = O.dequantize_accumulate_layers_alloc(off, n, pays, metas, wl, alpha, beta, out0)
    scale = np.abs(beta * out0.astype(np.float64))
    for p, m, w in zip(pays, metas, wl):
        scale += abs(alpha) * np.abs(O.dequantize_layers_alloc(off, n, p, m, w)
                                     .astype(np.float64))
    compare_values(out.cpu().numpy(), ref, scale)


@pytest.mark.parametrize("name", list(LAYOUTS))
@pytest.mark.parametrize("W", [1, 3, 16])
def test_aggregate_matches_the_oracle(dev, name, W):
    beta = 0.0 if W == 1 else 0.5
    dequantize_case(dev, LAYOUTS[name], W, seed=len(LAYOUTS[name]) + W,
                    alpha=1.0 / W, beta=beta)


def test_one_payload_is_exact(dev):
    """W = 1, alpha = 1, beta = 0: out is x_hat itself, bit for bit."""
    gq, torch = dev
    sizes = LAYOUTS["ragged"]
    off = _layout(sizes)
    n = int(off[-1])
    widths = [3, 2, 8, 4, 3, 3, 2, 3, 4, 8]
    g = WL.small_mixture(n, seed=12)
    p, m, _ = O.quantize_layers_alloc(off, g, None, widths, seed=12)
    x = O.dequantize_layers_alloc(off, n, p, m, widths)
    seg = np.asarray(O.alloc_segments(np.diff(off), widths), dtype=np.int64)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    gq.gq_dequantize_accumulate_layers_alloc(
        n, torch.from_numpy(off).cuda(), [torch.from_numpy(p).cuda()],
        [torch.from_numpy(m).cuda()],
        [torch.from_numpy(np.asarray(widths, dtype=np.int32)).cuda()],
        [torch.from_numpy(seg).cuda()], 1.0, 0.0, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), x.view(np.uint32))


def test_the_160_layer_gradient_whole(dev):
    """The layered 25.6M-element gradient with error feedback, widths from
    the device allocation at 3 bits per element: payload, maxima and
    residual bit for bit, then the aggregate of that payload."""
    gq, torch = dev
    sizes, _ = WL.ternary_layout()
    off = _layout(sizes)
    n, nl = int(off[-1]), off.size - 1
    g = WL.ternary_gradient(0)
    e = WL.ternary_gradient(1) * np.float32(0.05)
    OFF = torch.from_numpy(off).cuda()
    G = torch.from_numpy(g).cuda()
    E = torch.from_numpy(e.copy()).cuda()
    gd = gq.desc(0, 512, s=1)
    codes0, _ = gq.alloc_payload(gd, n)
    M0 = torch.empty(nl, dtype=torch.float32, device="cuda")
    gq.gq_quantize_layers(gd, OFF, G, None, 0, 0, codes0, M0)
    Wd = torch.empty(nl, dtype=torch.int32, device="cuda")
    Sg = torch.empty(nl + 1, dtype=torch.int64, device="cuda")
    gq.gq_allocate_layer_bits(n, OFF, M0, 3 * n, Wd, Sg)
    P = torch.empty(gq.gq_alloc_payload_bytes(n, nl), dtype=torch.uint8, device="cuda")
    M = torch.empty(nl, dtype=torch.float32, device="cuda")
    say(f"alloc quantize whole: n={n} nl={nl}")
    gq.gq_quantize_layers_alloc(OFF, G, E, Wd, Sg, 11, 3, P, M)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    gq.gq_dequantize_accumulate_layers_alloc(n, OFF, [P], [M], [Wd], [Sg], 1.0, 0.0, out)
    torch.cuda.synchronize()
    widths = Wd.cpu().numpy().tolist()
    assert len(set(widths)) > 1, "the allocation should mix widths here"
    rp, rm, re = O.quantize_layers_alloc(off, g, e, widths, seed=11, step=3)
    assert np.array_equal(P.cpu().numpy()[:rp.size], rp)
    assert np.array_equal(M.cpu().numpy(), rm)
    assert np.array_equal(E.cpu().numpy().view(np.uint32), re.view(np.uint32))
    x = O.dequantize_layers_alloc(off, n, rp, rm, widths)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), x.view(np.uint32))
