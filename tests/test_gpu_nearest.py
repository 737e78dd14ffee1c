"""GPU parity of deterministic rounding to the nearest level
(GQ_FLAG_NEAREST) against the oracle: the uniform scheme at every bucket
size, ORQ with and without clipping, ragged lengths, error feedback, dense
packing, and the full 25.6M-element layered ternary gradient with error
feedback.  Codes are compared byte for byte."""
import numpy as np
import pytest

import oracle as O
from communication_efficient_gradient_amd import workloads as WL
from tests.parity import compare_codes, compare_meta, say
from tests.test_gpu_small import check_quantize, dev, run_gpu, to_gq  # noqa: F401

pytestmark = pytest.mark.gpu

N = O.FLAG_NEAREST


@pytest.mark.parametrize("d", [64, 128, 256, 512, 1024, 2048, 8192, 32768])
@pytest.mark.parametrize("s", [1, 4, 127])
def test_uniform_nearest(dev, d, s):
    n = 2 * d + 37
    g = WL.small_mixture(n, seed=d + s, kind="laplace")
    desc = O.Desc(O.UNIFORM, d, s=s, flags=N)
    check_quantize(dev, desc, g, None, seed=d)
    e = WL.small_mixture(n, seed=d + s + 1) * np.float32(0.1)
    check_quantize(dev, desc, g, e, seed=d, step=3)


@pytest.mark.parametrize("n", [1, 3, 64, 65, 511, 4099])
def test_uniform_nearest_ragged_and_dense(dev, n):
    g = WL.small_mixture(n, seed=n, kind="heavy")
    for flags in (N, N | O.FLAG_DENSE):
        check_quantize(dev, O.Desc(O.UNIFORM, 64, s=2, flags=flags), g,
                       np.zeros_like(g), seed=n)


@pytest.mark.parametrize("d", [64, 256, 512, 2048, 8192])
@pytest.mark.parametrize("L", [3, 9])
@pytest.mark.parametrize("clip", [0, O.FLAG_CLIP])
def test_orq_nearest(dev, d, L, clip):
    n = 2 * d + 45
    g = WL.orq_gradient(n)
    check_quantize(dev, O.Desc(O.ORQ, d, L=L, flags=N | clip, clip_sigma=3.0),
                   g, None, seed=3)
    if d >= 512:
        check_quantize(dev, O.Desc(O.ORQ, d, L=L, flags=N | O.FLAG_DENSE | clip,
                                   clip_sigma=3.0), g, None, seed=3)


def test_seed_is_ignored_on_device(dev):
    n = 5 * 512 + 7
    g = WL.small_mixture(n, seed=77, kind="laplace")
    for desc in (O.Desc(O.UNIFORM, 512, s=1, flags=N),
                 O.Desc(O.ORQ, 512, L=5, flags=N)):
        c0, m0, _ = run_gpu(dev, desc, g, None, 0, 0)
        c1, m1, _ = run_gpu(dev, desc, g, None, 12345, 6)
        assert np.array_equal(c0, c1) and np.array_equal(m0, m1)


def test_ternary_nearest_ef_whole(dev):
    """The layered 25.6M-element ternary gradient, three error-feedback
    steps with deterministic rounding; codes, scales and residuals bit for
    bit."""
    gq, torch = dev
    d = O.Desc(O.UNIFORM, 512, s=1, flags=N)
    n = WL.TERNARY_N
    E = torch.zeros(n, device="cuda")
    e_ref = np.zeros(n, dtype=np.float32)
    codes, meta = gq.alloc_payload(to_gq(gq, d), n)
    for t in range(3):
        say(f"ternary nearest step {t}")
        g = WL.ternary_gradient(t)
        gq.gq_quantize(to_gq(gq, d), torch.from_numpy(g).cuda(), E, 2, t,
                       codes, meta)
        torch.cuda.synchronize()
        rc, rm, e_ref, _ = O.quantize(d, g, e_ref, seed=2, step=t)
        compare_codes(d, n, codes.cpu().numpy(), rc)
        compare_meta(d, meta.cpu().numpy().reshape(-1, 1), rm, exact=True)
        assert np.array_equal(E.cpu().numpy().view(np.uint32),
                              e_ref.view(np.uint32)), f"residual, step {t}"
