"""The seeded benchmark inputs are reproducible: the first and the last
2^24-element chunk of every workload hash to the SHA-256 digests recorded
in tests/golden/workload_digests.json (written by
``python -m communication_efficient_gradient_amd.workloads``, which draws
the inputs and hashes them; every chunk of every input is listed there).
numpy documents no stream stability for ``Generator`` across feature
releases, so the comparison is made under the numpy version the digests
were taken with."""
import json
import os

import numpy as np
import pytest

from communication_efficient_gradient_amd import workloads as WL

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "workload_digests.json")


@pytest.fixture(scope="module")
def digests():
    with open(GOLDEN) as f:
        d = json.load(f)
    if d["numpy"] != np.__version__:
        pytest.skip(f"digests taken with numpy {d['numpy']}, running {np.__version__}")
    assert d["chunk"] == WL.CHUNK
    return d


def _check(stream_chunks, make, n):
    """make(m, start) returns elements start .. start+m of the stream."""
    last = (n - 1) // WL.CHUNK
    for k in sorted({0, last}):
        lo = k * WL.CHUNK
        m = min(WL.CHUNK, n - lo)
        assert WL.chunk_sha256(make(m, lo)) == [stream_chunks[k]], f"chunk {k}"
    assert len(stream_chunks) == last + 1


def test_qsgd(digests):
    assert WL.chunk_sha256(WL.qsgd_gradient()) == digests["qsgd"]


def test_ternary_first_step(digests):
    assert WL.chunk_sha256(WL.ternary_gradient(0)) == digests["ternary"][0]


def test_orq_chunks(digests):
    _check(digests["orq"], lambda m, s: WL.orq_gradient(m, start=s), WL.ORQ_N)


def test_bingrad_chunks(digests):
    _check(digests["bingrad"], lambda m, s: WL.bingrad_gradient(m, start=s),
           WL.BINGRAD_N)


@pytest.mark.parametrize("w", [1, 8])
def test_worker_chunks(digests, w):
    _check(digests["workers"][w - 1],
           lambda m, s: WL.worker_gradient(w, m, start=s), WL.WORKERS_N)
