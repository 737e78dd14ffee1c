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
    assert bench.binopt_prune_ops() == 32
    f = bench.alu_fields(100.0, 10 ** 8, 1.0)
    assert abs(f["alu_frac"] - 1e10 / 1e-3 / bench.VALU_PEAK_LANE_OPS) < 1e-4


def test_ingest_counter_runs(tmp_path, monkeypatch):
    """`bench.py --ingest` turns two counter databases (FETCH_SIZE, WRITE_SIZE
    in KiB per dispatch) into bytes per launch, scaled by what the counters
    read for the known-size copy, per headline kernel and per BinGrad-b
    bucket size (the sort-free kernel and the sort kernel's pass summed)."""
    import sqlite3
    sys.path.insert(0, ROOT)
    import bench
    copy_kib = bench.COPY_BYTES / 1024
    rows = {
        "FETCH_SIZE": [("at::neg_kernel", copy_kib / 2),
                       (f"void gq::{bench.Headline.KERNEL}(long)", 1000.0),
                       ("void gq::k_stream_quant<1, 1, 64, 2>(long)", 7.0),
                       (f"void gq::{bench.Headline.AGG_KERNEL}(long)", 2000.0),
                       ("void gq::k_binopt_block<8192, true, true>(long)", 300.0),
                       ("void gq::k_binopt_block<8192, true, false>(long)", 3.0),
                       ("void gq::k_sort_quant<2, 1, 8192>(long)", 1.0),
                       ("void gq::k_wave_sort_quant<2, 1, 512, false, true>(long)", 400.0),
                       ("void gq::k_wave_sort_quant<3, 4, 512, true, true>(long)", 50.0),
                       ("void gq::k_wave_sort_quant<3, 4, 512, true, false>(long)", 0.5)],
        "WRITE_SIZE": [("at::neg_kernel", copy_kib),
                       (f"void gq::{bench.Headline.KERNEL}(long)", 100.0),
                       ("void gq::k_stream_quant<1, 1, 64, 2>(long)", 9.0),
                       (f"void gq::{bench.Headline.AGG_KERNEL}(long)", 200.0),
                       ("void gq::k_binopt_block<8192, true, true>(long)", 30.0),
                       ("void gq::k_binopt_block<8192, true, false>(long)", 0.3),
                       ("void gq::k_sort_quant<2, 1, 8192>(long)", 0.5),
                       ("void gq::k_wave_sort_quant<2, 1, 512, false, true>(long)", 40.0),
                       ("void gq::k_wave_sort_quant<3, 4, 512, true, true>(long)", 5.0),
                       ("void gq::k_wave_sort_quant<3, 4, 512, true, false>(long)", 0.05)],
    }
    dirs = []
    for cn, kv in rows.items():
        d = tmp_path / cn
        d.mkdir()
        con = sqlite3.connect(str(d / "run.db"))
        con.execute("create table counters_collection "
                    "(kernel_name text, counter_name text, value real)")
        for name, v in kv:
            con.execute("insert into counters_collection values (?, ?, ?)", (name, cn, v))
        con.commit()
        con.close()
        dirs.append(str(d))
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.ingest(dirs)
    import json
    t = json.loads(out.read_text())
    assert t["_calibration"]["fetch_scale"] == 2.0
    assert t["_calibration"]["write_scale"] == 1.0
    assert t[bench.Headline.KEY]["bytes_per_launch"] == 1000 * 2048 + 100 * 1024
    assert t[bench.Headline.AGG_KEY]["bytes_per_launch"] == 2000 * 2048 + 200 * 1024
    assert t["bin_opt_ef_d8192_n1B"]["bytes_per_launch"] == 301 * 2048 + 30.5 * 1024
    assert t["bin_opt_ef_d512_n1B"]["bytes_per_launch"] == 400 * 2048 + 40 * 1024
    assert "bin_opt_ef_d2048_n1B" not in t
    # ORQ: the whole-bucket kernel of each (L, bisection) seen in the runs
    assert t["orq_L9_bisect_d512_n100M"]["bytes_per_launch"] == 50 * 2048 + 5 * 1024
    assert "orq_L5_d512_n100M" not in t
