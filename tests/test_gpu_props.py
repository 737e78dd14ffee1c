"""Properties of the HIP path that hold at any size, checked on the GPU's own
output (no oracle arithmetic involved):

* unbiasedness of the random rounding, E[Q(x)] = x, over many seeds, with the
  exact two-point variance (b - x)(x - a) as the yardstick ("Gradient
  Quantization" glossary, Stochastic Quantization bullet);
* the 0.7-between-0-and-1 example of the same bullet, on the device;
* error feedback carries state only in the residual (Philox is counter
  based), so five steps run straight equal two steps, a round trip of the
  residual through host memory, then three more steps, bit for bit;
* a missing worker: aggregating the W - 1 payloads that arrived with
  alpha = 1/(W - 1) is their average, and the average of W identical
  payloads is that payload's value (to fp32 summation error).
"""
import numpy as np
import pytest

from communication_efficient_gradient_amd import workloads as WL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from communication_efficient_gradient_amd import gq
    return gq, torch


def _dequant(gq, torch, d, n, codes, meta):
    out = torch.empty(n, device="cuda")
    gq.gq_dequantize_accumulate(d, n, [codes], [meta], 1.0, 0.0, out)
    return out


@pytest.mark.parametrize("scheme,s,L", [(0, 1, 5), (0, 4, 5), (3, 5, 5),
                                        (3, 9, 9)])
def test_unbiased_over_seeds(dev, scheme, s, L):
    gq, torch = dev
    n, seeds = 1024, 2048
    d = gq.desc(scheme, 512, s=s, levels=L)
    g = WL.small_mixture(n, seed=31, kind="laplace")
    G = torch.from_numpy(g).cuda()
    codes, meta = gq.alloc_payload(d, n)
    acc = torch.zeros(n, dtype=torch.float64, device="cuda")
    acc2 = torch.zeros(n, dtype=torch.float64, device="cuda")
    for seed in range(seeds):
        gq.gq_quantize(d, G, None, seed, 0, codes, meta)
        x = _dequant(gq, torch, d, n, codes, meta).double()
        acc += x
        acc2 += x * x
    torch.cuda.synchronize()
    mean = (acc / seeds).cpu().numpy()
    var = (acc2 / seeds).cpu().numpy() - mean ** 2
    x = g.astype(np.float64)
    # exact two-point variance around x from the levels the GPU used
    gq.gq_quantize(d, G, None, 0, 0, codes, meta)
    m = meta.cpu().numpy()
    if scheme == 0:
        delta = np.repeat(m.astype(np.float64) / s, 512)[:n]
        lo = np.floor(np.abs(x) / delta) * delta
        a, b = lo, lo + delta
        v = (b - np.abs(x)) * (np.abs(x) - a)
    else:
        lv = m.reshape(-1, L).astype(np.float64)
        v = np.zeros(n)
        for j in range(lv.shape[0]):
            sl = slice(512 * j, min(n, 512 * (j + 1)))
            idx = np.clip(np.searchsorted(lv[j], x[sl], side="right") - 1, 0, L - 2)
            a, b = lv[j][idx], lv[j][idx + 1]
            v[sl] = np.maximum((b - x[sl]) * (x[sl] - a), 0.0)
    live = v > 0
    z = (mean[live] - x[live]) / np.sqrt(v[live] / seeds)
    assert np.all(np.abs(z) < 6.5), np.abs(z).max()
    chi2 = float((z ** 2).sum())
    k = int(live.sum())
    assert abs(chi2 - k) < 6 * np.sqrt(2 * k), (chi2, k)
    # the empirical variance matches (b - x)(x - a) on average
    assert abs(var[live].sum() / v[live].sum() - 1.0) < 0.1
    # values sitting on a level never move
    assert np.all(np.abs(mean[~live] - x[~live]) <= 1e-7 * np.abs(x[~live]) + 1e-30)


def test_point_seven_on_device(dev):
    """Ternary s=1 on a bucket whose max-abs is 1: 0.7 rounds up to 1 with
    probability 0.7 (to within the 2^-24 resolution of u)."""
    gq, torch = dev
    n = 512 * 512
    g = np.full(n, 0.7, dtype=np.float32)
    g[::512] = 1.0
    d = gq.desc(0, 512, s=1)
    G = torch.from_numpy(g).cuda()
    codes, meta = gq.alloc_payload(d, n)
    ups = 0
    trials = 0
    for seed in range(8):
        gq.gq_quantize(d, G, None, seed, 0, codes, meta)
        x = _dequant(gq, torch, d, n, codes, meta).cpu().numpy()
        body = np.ones(n, bool)
        body[::512] = False
        assert set(np.unique(x[body]).tolist()) <= {0.0, 1.0}
        ups += int((x[body] == 1.0).sum())
        trials += int(body.sum())
    p = float(np.float32(0.7))
    sd = np.sqrt(p * (1 - p) / trials)
    assert abs(ups / trials - p) < 5 * sd, (ups / trials, p, sd)


@pytest.mark.parametrize("scheme", [0, 2, 3])
def test_error_feedback_resume_bit_exact(dev, scheme):
    gq, torch = dev
    n = 20 * 512 + 77
    d = gq.desc(scheme, 512, s=1, levels=5, flags=0)
    grads = [torch.from_numpy(WL.small_mixture(n, seed=40 + t, kind="laplace")).cuda()
             for t in range(5)]
    codes, meta = gq.alloc_payload(d, n)

    def run(e, steps):
        outs = []
        for t in steps:
            gq.gq_quantize(d, grads[t], e, 9, t, codes, meta)
            outs.append((codes.clone(), meta.clone()))
        return outs

    e1 = torch.zeros(n, device="cuda")
    straight = run(e1, range(5))
    e2 = torch.zeros(n, device="cuda")
    first = run(e2, range(2))
    saved = e2.cpu().numpy().copy()          # checkpoint: the residual only
    e3 = torch.from_numpy(saved).cuda()      # resume in a fresh buffer
    rest = run(e3, range(2, 5))
    torch.cuda.synchronize()
    for (c1, m1), (c2, m2) in zip(straight, first + rest):
        assert torch.equal(c1, c2) and torch.equal(m1.view(torch.int32), m2.view(torch.int32))
    assert torch.equal(e1.view(torch.int32), e3.view(torch.int32))


def test_missing_worker_and_identical_payloads(dev):
    gq, torch = dev
    n, W = 6 * 512 + 3, 8
    d = gq.desc(0, 512, s=127)
    payloads = []
    for w in range(W):
        G = torch.from_numpy(WL.small_mixture(n, seed=60 + w)).cuda()
        c, m = gq.alloc_payload(d, n)
        gq.gq_quantize(d, G, None, w + 1, 0, c, m)
        payloads.append((c, m))
    # worker 3 dropped out: average the seven that arrived
    arrived = [p for i, p in enumerate(payloads) if i != 3]
    out = torch.empty(n, device="cuda")
    gq.gq_dequantize_accumulate(d, n, [c for c, _ in arrived],
                                [m for _, m in arrived], 1.0 / 7, 0.0, out)
    xs = torch.stack([_dequant(gq, torch, d, n, c, m).double() for c, m in arrived])
    ref = xs.sum(0) / 7
    scale = xs.abs().sum(0) / 7
    assert torch.all((out.double() - ref).abs() <= 1e-6 * scale + 1e-37)
    # W identical payloads average to that payload (fp32 sums of equal terms
    # round, so to within the aggregation tolerance)
    c, m = payloads[0]
    gq.gq_dequantize_accumulate(d, n, [c] * W, [m] * W, 1.0 / W, 0.0, out)
    x0 = _dequant(gq, torch, d, n, c, m)
    torch.cuda.synchronize()
    assert torch.all((out - x0).abs() <= 1e-6 * x0.abs())
