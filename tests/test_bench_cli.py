"""bench.py's command line on the CPU: more than one GPU is refused with a
message and exit status 2 before anything is imported from torch or the
library, and the algorithmic byte counts it reports follow the formulas
(quantize: g, e in and out, codes, meta; dequantize-accumulate: W payloads
and the output)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes():
    sys.path.insert(0, ROOT)
    import bench
    n = 25_600_000
    # ternary + EF, d = 512: 12 B of fp32 streams, 2 bits, one scale per bucket
    assert bench.quant_bytes(2, 1, 512, n, True) == 12 * n + n // 4 + 4 * 50_000
    # INT8 W = 8 average over 256M: 8 payloads of codes + scales, then out
    m = 256_000_000
    assert bench.deq_bytes(8, 1, 512, m, 8, 0.0) == 8 * (m + 4 * 500_000) + 4 * m
    # beta != 0 reads the output too; a ragged last bucket still has a scale
    assert bench.deq_bytes(4, 1, 512, 1000, 1, 0.5) == 500 + 4 * 2 + 8 * 1000


def test_alu_op_counts():
    """The ALU-bound kernels' algorithmic lane-operations per element follow
    their stated formulas: a bitonic sort of d = 512 makes 22.5
    compare-exchanges per element (two ops each); ORQ-9 rescans the bucket
    in each of its 7 greedy steps (10 ops per element per step)."""
    sys.path.insert(0, ROOT)
    import bench
    assert bench.sort_ops(512) == 45.0
    assert bench.sort_ops(128) == 28.0
    assert bench.orq_ops(9, 512) == 45 + 70 + 3 + 20 + 10
    assert bench.orq_ops(5, 512, clip=True) == 45 + 4 + 30 + 2 + 20 + 10
    # bisection: L = 9 takes three rounds, L = 5 two
    assert bench.orq_ops(9, 512, bisect=True) == 45 + 30 + 3 + 20 + 10
    assert bench.orq_ops(5, 512, bisect=True) == 45 + 20 + 2 + 20 + 10
    assert bench.binopt_ops(512) == 1 + 45 + 2 + 6 + 1 + 4
    assert bench.binopt_prune_ops() == 36
    f = bench.alu_fields(100.0, 10 ** 8, 1.0)
    assert abs(f["alu_frac"] - 1e10 / 1e-3 / bench.VALU_PEAK_LANE_OPS) < 1e-4
