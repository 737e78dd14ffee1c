"""GPU parity on small inputs: every scheme, every bucket size, ragged tails.

The HIP library (through its C ABI) against the CPU oracle on the same seeded
inputs, element by element.  Sizes span several buckets and a partial last
bucket; the oracle finishes each case in milliseconds.
"""
import numpy as np
import pytest

import oracle as O
from communication_efficient_gradient_amd import workloads as WL
from tests.parity import (compare_codes, compare_meta, compare_values,
                          bucket_mask, say)

pytestmark = pytest.mark.gpu

BUCKETS = [64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768]


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from communication_efficient_gradient_amd import gq
    return gq, torch


def to_gq(gq, d: O.Desc):
    return gq.desc(d.scheme, d.d, d.s, d.L, d.flags, d.clip_sigma)


def run_gpu(dev, d: O.Desc, g, e, seed, step):
    gq, torch = dev
    gd = to_gq(gq, d)
    G = torch.from_numpy(g).cuda()
    E = None if e is None else torch.from_numpy(e.copy()).cuda()
    codes, meta = gq.alloc_payload(gd, g.size)
    codes.fill_(0xAB)  # poison: every byte up to code_bytes must be written
    gq.gq_quantize(gd, G, E, seed, step, codes, meta)
    torch.cuda.synchronize()
    return (codes.cpu().numpy(), meta.cpu().numpy().reshape(-1, d.k),
            None if E is None else E.cpu().numpy())


def gpu_deq(dev, d: O.Desc, n, codes_list, meta_list, alpha=1.0, beta=0.0,
            out=None):
    gq, torch = dev
    gd = to_gq(gq, d)
    C = [torch.from_numpy(np.ascontiguousarray(c)).cuda() for c in codes_list]
    M = [torch.from_numpy(np.ascontiguousarray(m.ravel())).cuda() for m in meta_list]
    if out is None:
        O_ = torch.full((n,), float("nan"), device="cuda")
    else:
        O_ = torch.from_numpy(out.copy()).cuda()
    gq.gq_dequantize_accumulate(gd, n, C, M, alpha, beta, O_)
    torch.cuda.synchronize()
    return O_.cpu().numpy()


def check_quantize(dev, d: O.Desc, g, e, seed=1, step=0):
    say(f"case scheme={d.scheme} d={d.d} s={d.s} L={d.L} flags={d.flags} "
        f"n={g.size} ef={e is not None} seed={seed} step={step}")
    n = g.size
    rc, rm, re_, tie = O.quantize(d, g, e, seed=seed, step=step)
    gc, gm, ge = run_gpu(dev, d, g, e, seed, step)
    exact = d.scheme in (O.UNIFORM, O.BIN_SIGN)
    bad = compare_codes(d, n, gc, rc, tie, exact=exact)
    if d.scheme == O.UNIFORM:
        compare_meta(d, gm, rm, exact=True)
    elif d.scheme == O.ORQ and not d.flags & O.FLAG_CLIP:
        compare_meta(d, gm, rm, skip=bad, exact=False)
        keep = np.ones(rm.shape[0], bool)
        keep[bad] = False
        assert np.array_equal(gm[keep], rm[keep])
    else:
        compare_meta(d, gm, rm, skip=bad)
    if e is not None:
        p = (g + e).astype(np.float64)
        m = bucket_mask(d, n, bad)
        scale = np.maximum(np.abs(p), np.abs(p - re_))
        lvl_tol = 1e-5 * np.abs(p - re_)
        compare_values(ge[m], re_[m], scale[m], exact=(d.scheme == O.UNIFORM),
                       extra=lvl_tol[m])
    # dequantize (W = 1) reproduces the oracle's x-hat exactly
    xg = gpu_deq(dev, d, n, [gc], [gm])
    xr = O.dequantize(d, n, gc, gm)
    compare_values(xg, xr, np.abs(xr), exact=True)
    return bad


@pytest.mark.parametrize("d", BUCKETS)
@pytest.mark.parametrize("s", [1, 4, 127])
def test_uniform_every_bucket(dev, d, s):
    n = 3 * d + 37
    g = WL.small_mixture(n, seed=d + s, kind="laplace")
    check_quantize(dev, O.Desc(O.UNIFORM, d, s=s), g, None, seed=d)
    e = WL.small_mixture(n, seed=d + s + 1) * np.float32(0.1)
    check_quantize(dev, O.Desc(O.UNIFORM, d, s=s), g, e, seed=d, step=3)


@pytest.mark.parametrize("s", [2, 3, 5, 7, 8, 100])
@pytest.mark.parametrize("n", [1, 2, 3, 5, 63, 64, 65, 511, 513, 1027, 4099])
def test_uniform_ragged(dev, s, n):
    g = WL.small_mixture(n, seed=n * 7 + s, kind="heavy")
    e = WL.small_mixture(n, seed=n * 7 + s + 1) * np.float32(0.01)
    check_quantize(dev, O.Desc(O.UNIFORM, 64, s=s), g, e, seed=s)


def test_uniform_edge_values(dev):
    d = 64
    g = np.zeros(7 * d + 3, dtype=np.float32)
    g[d:2 * d] = -0.0
    g[2 * d:3 * d] = 3.0
    g[3 * d:4 * d] = np.float32(1e-44)
    g[3 * d + 5] = np.float32(-3e-45)
    g[4 * d:5 * d] = np.linspace(-1, 1, d, dtype=np.float32)
    g[5 * d:6 * d] = np.float32(3e38) * np.sign(np.arange(d) - 31.5).astype(np.float32)
    g[6 * d:] = WL.small_mixture(d + 3, seed=5, kind="wide")
    for s in (1, 4, 127):
        check_quantize(dev, O.Desc(O.UNIFORM, d, s=s), g, None, seed=9)
        check_quantize(dev, O.Desc(O.UNIFORM, d, s=s), g, np.zeros_like(g), seed=9)


@pytest.mark.parametrize("d", BUCKETS)
@pytest.mark.parametrize("scheme", [O.BIN_SIGN, O.BIN_OPT])
def test_two_level_every_bucket(dev, d, scheme):
    n = 3 * d + 21
    g = WL.bingrad_gradient(n)
    e = WL.small_mixture(n, seed=d) * np.float32(0.001)
    check_quantize(dev, O.Desc(scheme, d), g, None)
    check_quantize(dev, O.Desc(scheme, d), g, e, step=1)


@pytest.mark.parametrize("n", [1, 2, 3, 17, 64, 65, 130, 1000])
def test_two_level_ragged_and_degenerate(dev, n):
    for kind in ("normal", "ints", "positive"):
        g = WL.small_mixture(n, seed=n, kind=kind)
        for scheme in (O.BIN_SIGN, O.BIN_OPT):
            check_quantize(dev, O.Desc(scheme, 64), g, np.zeros_like(g))
    g = np.zeros(200, dtype=np.float32)
    g[64:128] = 2.5
    g[128:192] = -0.0
    for scheme in (O.BIN_SIGN, O.BIN_OPT):
        check_quantize(dev, O.Desc(scheme, 64), g, np.zeros_like(g))


@pytest.mark.parametrize("d", [64, 512, 1024, 4096, 16384, 32768])
def test_binopt_large_bucket_edge_cases(dev, d):
    """BinGrad-b buckets that take every branch of the split selection, in
    the register-sort kernel (d <= 512) and the sort-free search (d >=
    1024): no split (one value), signed zeros, small integers (ties the
    search cannot narrow: the bucket goes to the sort-based path), cluster
    sums that cancel (the compensated recomputation), scales outside the
    search's fixed-point range (straight to the sort), evenly spread
    values, and a ragged tail of 100 values."""
    rng = np.random.default_rng(d)
    zeros = np.where(rng.random(d) < 0.5, -0.0, 0.0).astype(np.float32)
    zeros[rng.choice(d, 40, replace=False)] = rng.standard_normal(40).astype(np.float32)
    v = rng.standard_normal(d // 2 - 8).astype(np.float32)
    cancel = np.concatenate([v, -v, np.full(16, 100.0, np.float32)])
    cancel[0] += np.float32(1e-3)
    spread = np.linspace(-1, 1, d, dtype=np.float32)
    parts = [np.full(d, 2.5, np.float32), zeros,
             rng.integers(-3, 4, d).astype(np.float32),
             rng.permutation(cancel),
             (rng.standard_normal(d) * 1e30).astype(np.float32),
             (rng.standard_normal(d) * 1e-30).astype(np.float32),
             rng.permutation(spread),
             rng.standard_normal(100).astype(np.float32)]
    g = np.concatenate(parts)
    check_quantize(dev, O.Desc(O.BIN_OPT, d), g, None)
    check_quantize(dev, O.Desc(O.BIN_OPT, d), g, np.zeros_like(g), step=1)


@pytest.mark.parametrize("d", [64, 128, 256, 512, 1024, 2048, 4096])
@pytest.mark.parametrize("L", [2, 3, 5, 9, 16])
@pytest.mark.parametrize("clip", [0, 1])
def test_orq_every_bucket(dev, d, L, clip):
    n = 2 * d + 45
    g = WL.orq_gradient(n)
    d_ = O.Desc(O.ORQ, d, L=L, flags=clip, clip_sigma=3.0)
    check_quantize(dev, d_, g, None, seed=3)
    e = WL.small_mixture(n, seed=L) * np.float32(1e-4)
    check_quantize(dev, d_, g, e, seed=3, step=2)


@pytest.mark.parametrize("d", [8192, 16384, 32768])
def test_orq_large_buckets(dev, d):
    g = WL.orq_gradient(d + 1000)
    check_quantize(dev, O.Desc(O.ORQ, d, L=5), g, None, seed=4)
    check_quantize(dev, O.Desc(O.ORQ, d, L=9, flags=1), g, None, seed=4)


@pytest.mark.parametrize("n", [1, 5, 64, 100, 777])
def test_orq_ragged_and_few_values(dev, n):
    for kind in ("ints", "normal"):
        g = WL.small_mixture(n, seed=n + 1, kind=kind)
        for L in (3, 9):
            check_quantize(dev, O.Desc(O.ORQ, 64, L=L), g, np.zeros_like(g))


@pytest.mark.parametrize("scheme,s,L", [(O.UNIFORM, 127, 5), (O.UNIFORM, 4, 5),
                                        (O.UNIFORM, 1, 5), (O.UNIFORM, 3, 5),
                                        (O.BIN_SIGN, 4, 5), (O.BIN_OPT, 4, 5),
                                        (O.ORQ, 4, 9), (O.ORQ, 4, 5),
                                        (O.ORQ, 4, 3), (O.ORQ, 4, 2)])
@pytest.mark.parametrize("W", [1, 2, 3, 8, 16])
def test_dequantize_accumulate(dev, scheme, s, L, W):
    n = 3 * 512 + 19
    d = O.Desc(scheme, 512, s=s, L=L)
    cl, ml = [], []
    for w in range(W):
        g = WL.small_mixture(n, seed=100 + w)
        c, m, _, _ = O.quantize(d, g, seed=w)
        cl.append(c)
        ml.append(m)
    out0 = WL.small_mixture(n, seed=7)
    xs = [O.dequantize(d, n, c, m).astype(np.float64) for c, m in zip(cl, ml)]
    absum = np.sum([np.abs(x) for x in xs], axis=0)
    for alpha, beta in [(1.0, 0.0), (1.0 / W, 0.0), (0.3, 1.0), (1.0, -0.5)]:
        say(f"deq scheme={scheme} W={W} alpha={alpha} beta={beta}")
        got = gpu_deq(dev, d, n, cl, ml, alpha, beta, out0 if beta else None)
        ref = O.dequantize_accumulate(d, n, cl, ml, alpha, beta,
                                      out0 if beta else None)
        scale = abs(beta) * np.abs(out0.astype(np.float64)) + abs(alpha) * absum
        compare_values(got, ref, scale, exact=(W == 1 and alpha == 1.0 and beta == 0.0))


@pytest.mark.parametrize("scheme,s,L", [(O.UNIFORM, 127, 5), (O.UNIFORM, 4, 5),
                                        (O.ORQ, 4, 9)])
@pytest.mark.parametrize("bucket", [64, 512, 8192])
@pytest.mark.parametrize("W", [1, 5, 16])
def test_dequantize_accumulate_tiles(dev, scheme, s, L, bucket, W):
    """4- and 8-bit codes over several 4096-element tiles and a ragged tail:
    per-tile step tables of up to 64 buckets, whole and partial wave runs."""
    n = 6 * 4096 + 777
    d = O.Desc(scheme, bucket, s=s, L=L)
    cl, ml = [], []
    for w in range(W):
        g = WL.small_mixture(n, seed=300 + w)
        c, m, _, _ = O.quantize(d, g, seed=w + 1)
        cl.append(c)
        ml.append(m)
    xs = [O.dequantize(d, n, c, m).astype(np.float64) for c, m in zip(cl, ml)]
    absum = np.sum([np.abs(x) for x in xs], axis=0)
    for alpha, beta in [(1.0, 0.0), (1.0 / W, 0.0), (0.5, 2.0)]:
        say(f"deq tiles scheme={scheme} d={bucket} W={W} alpha={alpha} beta={beta}")
        out0 = WL.small_mixture(n, seed=9)
        got = gpu_deq(dev, d, n, cl, ml, alpha, beta, out0 if beta else None)
        ref = O.dequantize_accumulate(d, n, cl, ml, alpha, beta,
                                      out0 if beta else None)
        scale = abs(beta) * np.abs(out0.astype(np.float64)) + abs(alpha) * absum
        compare_values(got, ref, scale,
                       exact=(W == 1 and alpha == 1.0 and beta == 0.0))


@pytest.mark.parametrize("scheme,s,L", [
    (O.UNIFORM, 1, 5), (O.UNIFORM, 127, 5), (O.UNIFORM, 2, 5), (O.BIN_OPT, 4, 5),
    # A run of this case once left the GPU faulted (the build under test then
    # recomputed the coding pass's addresses; that change is out again).  No
    # cause has been shown, so the case stays off the GPU until one is.
    pytest.param(O.ORQ, 4, 9, marks=pytest.mark.skip(
        reason="GPU fault seen once on this case; cause not shown"))])
def test_error_feedback_standalone_equals_fused(dev, scheme, s, L):
    gq, torch = dev
    n = 5 * 512 + 77
    d = O.Desc(scheme, 512, s=s, L=L, flags=1 if scheme == O.ORQ else 0)
    g = WL.small_mixture(n, seed=1)
    e = WL.small_mixture(n, seed=2) * np.float32(0.1)
    gc, gm, ge = run_gpu(dev, d, g, e, 5, 1)
    gd = to_gq(gq, d)
    E = torch.from_numpy(e.copy()).cuda()
    gq.gq_error_feedback(gd, torch.from_numpy(g).cuda(), E,
                         torch.from_numpy(gc).cuda(),
                         torch.from_numpy(gm.ravel().copy()).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(E.cpu().numpy().view(np.uint32), ge.view(np.uint32))
    ref = O.error_feedback(d, g, e, gc, gm)
    assert np.array_equal(ref.view(np.uint32), ge.view(np.uint32))


@pytest.mark.parametrize("scheme", [O.UNIFORM, O.BIN_SIGN, O.BIN_OPT, O.ORQ])
def test_select_levels_matches_quantize(dev, scheme):
    gq, torch = dev
    n = 9 * 512 + 5
    d = O.Desc(scheme, 512, s=4, L=9)
    g = WL.orq_gradient(n)
    e = WL.small_mixture(n, seed=3) * np.float32(1e-4)
    _, gm, _ = run_gpu(dev, d, g, e, 1, 0)
    gd = to_gq(gq, d)
    meta = torch.empty(gm.size, device="cuda")
    gq.gq_select_levels(gd, torch.from_numpy(g).cuda(),
                        torch.from_numpy(e).cuda(), meta)
    torch.cuda.synchronize()
    assert np.array_equal(meta.cpu().numpy(), gm.ravel())
    rm, tie = O.select_levels(d, g, e)
    compare_meta(d, gm, rm, skip=np.nonzero(tie)[0],
                 exact=(scheme == O.UNIFORM))


def test_deterministic_repeat(dev):
    for d in (O.Desc(O.UNIFORM, 512, s=1), O.Desc(O.BIN_OPT, 2048),
              O.Desc(O.ORQ, 512, L=9, flags=1)):
        g = WL.orq_gradient(20 * d.d + 3)
        e = WL.small_mixture(g.size, seed=4) * np.float32(1e-4)
        a = run_gpu(dev, d, g, e, 7, 2)
        b = run_gpu(dev, d, g, e, 7, 2)
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def _bingrad_after_ef_steps(d: int, buckets, steps: int):
    """Buckets `buckets` of the 1B bingrad gradient (bucket indices counted
    from element 2^24 on, inside its second and third chunks of 2^24 values)
    and the residuals the oracle's own BinGrad-b + error-feedback steps
    leave on them: (g, [e_0 = 0, e_1, ..., e_steps])."""
    chunk = WL.bingrad_gradient(2 * WL.CHUNK, start=WL.CHUNK)
    g = np.concatenate([chunk[b * d:(b + 1) * d] for b in buckets])
    es = [np.zeros_like(g)]
    for t in range(steps):
        _, _, e_next, _ = O.quantize(O.Desc(O.BIN_OPT, d), g, es[-1], seed=0, step=t)
        es.append(e_next)
    return g, es


def test_binopt_after_ef_steps(dev):
    """BinGrad-b on buckets that a few error-feedback steps have shaped so
    that near-maximal splits stay many (on the GPU's own trajectory the
    split search's levels ran out there with 65 to 208 values left): each
    step's quantize against the oracle, the residuals being the oracle's."""
    d = 32768
    g, es = _bingrad_after_ef_steps(d, [436, 437, 438, 564, 662, 663], 4)
    for t, e in enumerate(es):
        check_quantize(dev, O.Desc(O.BIN_OPT, d), g, e, step=t)
