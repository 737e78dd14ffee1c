#!/usr/bin/env python3
"""Throughput of bucketed stochastic gradient quantization with error feedback
on one MI355X.

A step of the headline workload is the whole data-parallel path for eight
simulated workers on one GPU: each worker's 256M-element fp32 gradient goes
through one fused INT8 (s = 127) error-feedback quantize (p = g + e, per-bucket
max-abs scale with d = 512, Philox random rounding, 8-bit packing, residual
write-back), then the receiving side unpacks, dequantizes and averages the
eight payloads into one fp32 buffer (W = 8, alpha = 1/8).  The eight seeded
gradients are resident in HBM and every worker carries its residual from step
to step.

Printed: ONE JSON line with the whole-job throughput (GB/s of fp32 gradient
through quantize + aggregate), the roofline of the dominant kernel (the fused
INT8 quantizer) from HIP events recorded around every launch of the timed
region on the launch stream, the CPU oracle timed on the host as a baseline,
and one entry per other kernel/workload (QSGD latency, ternary + EF on the
layered 25.6M gradient, ORQ-5/9, BinGrad-b / sign over the bucket sweep, and
the variants).

    python bench.py [--steps K] [--warmup W] [--suite main|all]
    python bench.py --counters          # short run for rocprofv3 --pmc
    python bench.py --ingest DIR        # turn two --pmc runs into traffic
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("GB/s of fp32 gradient quantized+packed (and dequant+accumulated); "
          "% HBM peak")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
# VALU peak in lane-operations per second for 32-bit and fp64 add / multiply /
# fused multiply-add without packed fp32: 256 CUs x 4 SIMDs x 16 lanes x
# 2.4 GHz = 39.3 T (one wave64 instruction per CU per cycle).  The published
# 157.3 TFLOP/s fp32 figure counts packed fp32 (two lanes' worth per
# instruction) and two flops per FMA; this library is built without packed
# fp32.  The rate was measured on the GPU with independent chains of each
# instruction (see the measured-peaks table in the design notes).
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
PARITY_FILE = os.path.join(ROOT, "profiles", "parity_full.json")
_CSRC = "communication_efficient_gradient_amd/csrc/"
# the sources (and build flags) each measured kernel is compiled from
KERNEL_SOURCES = {
    "k_stream_quant": [_CSRC + "common.hpp", _CSRC + "stream_quant.hip",
                       "communication_efficient_gradient_amd/build.py"],
    "k_deq_acc": [_CSRC + "common.hpp", _CSRC + "deq.hip",
                  "communication_efficient_gradient_amd/build.py"],
    "bin_opt": [_CSRC + "common.hpp", _CSRC + "sort_quant.hip",
                _CSRC + "binopt_quant.hip",
                "communication_efficient_gradient_amd/build.py"],
    "orq": [_CSRC + "common.hpp", _CSRC + "sort_quant.hip",
            "communication_efficient_gradient_amd/build.py"],
}
ORQ_TRAFFIC = ((5, False), (9, False), (5, True), (9, True))  # (L, bisection)


def orq_traffic_key(L: int, bisect: bool) -> str:
    return f"orq_L{L}{'_bisect' if bisect else ''}_d512_n100M"
BINGRAD_BUCKETS = (128, 512, 2048, 8192, 32768)
COPY_BYTES = 1 << 29           # known-size copy for counter calibration


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------- algorithmic bytes --
def quant_bytes(bits: int, k: int, d: int, n: int, ef: bool) -> int:
    """HBM bytes a quantize launch must move: g (+ e in, e out), codes, meta."""
    nb = (n + d - 1) // d
    return 4 * n + (8 * n if ef else 0) + (n * bits + 7) // 8 + 4 * k * nb


def deq_bytes(bits: int, k: int, d: int, n: int, W: int, beta: float) -> int:
    """HBM bytes of dequantize-accumulate: W payloads, out (+ out read)."""
    nb = (n + d - 1) // d
    per = (n * bits + 7) // 8 + 4 * k * nb
    return W * per + 4 * n + (4 * n if beta != 0.0 else 0)


# ------------------------------------------------------ algorithmic ops --
# Lane-operations per element of the ALU-bound kernels' algorithms (each
# fp32 / int32 / fp64 add, multiply, fused multiply-add, min, max, compare,
# select, shift or logic op counts one; a division counts one), as the design
# notes derive them.  Shared parts:
#   bitonic sort of a d-bucket: log2 d (log2 d + 1) / 4 compare-exchanges per
#     element, two ops each (min and max);
#   Philox4x32-10: 10 rounds x (2 multiply-low + 2 multiply-high + 2 three-
#     input xor + 2 key adds) per 4 elements = 20 per element;
#   random rounding between two levels and packing: 10 per element.
PHILOX_OPS = 20
ROUND_PACK_OPS = 10


def _log2(d: int) -> int:
    return d.bit_length() - 1


def sort_ops(d: int) -> float:
    lg = _log2(d)
    return 2 * lg * (lg + 1) / 4


def orq_ops(L: int, d: int, clip: bool = False, bisect: bool = False) -> float:
    """ORQ-L: sort; optional clip (square-accumulate, two clamps: 4); each
    greedy step rescans the bucket (two fp64 prefix sums of (y - a) and
    (b - y): 4, the gain (b - c) A + (c - a) B: 5, the argmax compare: 1 =
    10 per element), L - 2 steps (bisection: ceil(log2(L - 1)) rounds of one
    rescan each); level search log2 L compares; Philox; rounding and
    packing."""
    steps = (L - 2) if not bisect else (L - 2).bit_length()
    return (sort_ops(d) + (4 if clip else 0) + 10 * steps + _log2(L)
            + PHILOX_OPS + ROUND_PACK_OPS)


def binopt_ops(d: int) -> float:
    """BinGrad-b with error feedback: EF add (1); sort; one fp64 prefix sum
    (convert + add: 2); the split objective P^2/k + (S - P)^2/(n - k) (one
    subtract, two multiplies, two divides, one add: 6) and the argmax compare
    (1); threshold compare, level select, residual subtract, pack (4)."""
    return 1 + sort_ops(d) + 2 + 6 + 1 + 4


def binopt_prune_ops() -> float:
    """BinGrad-b with error feedback by the sort-free split search (buckets of
    1024 and more): EF add (1); order-preserving key (2); bucket minimum,
    maximum, sum and absolute sum (4); the first level's bin, fixed-point
    value and LDS add for every element (5); the second level's range test
    and insertion, which reaches nearly every element (7); one more level's
    range test (2; 64 bins per level leave 2-3 levels); the exact stage's
    sums below the ranges and survivor test (7); threshold compare, level
    select, residual subtract, pack (4).  The bin evaluation and the
    survivor sort are per bucket, not per element."""
    return 1 + 2 + 4 + 5 + 7 + 2 + 7 + 4


def topk_ops(d: int, K: int) -> float:
    """Top-K with quantization and error feedback: EF add and |p| key (2);
    a 31-round bitwise selection of the K-th largest key (compare + count
    per round: 62); rank of the kept (2); residual (2); the kept elements'
    Philox, rounding and packing (K / d of 30)."""
    return 2 + 62 + 2 + 2 + (K / d) * (PHILOX_OPS + ROUND_PACK_OPS)


def elias_encode_ops() -> float:
    """Elias gamma encode: code unpack (2), codeword length (3), the count
    pass's sum (1), the record pass's prefix sum (1) and bit placement
    (shift, or, and word split: 4)."""
    return 11.0


def alu_fields(ops_per_element: float, n: int, ms: float) -> dict:
    achieved = ops_per_element * n / (ms * 1e-3)
    return {"alu_ops_per_element": round(ops_per_element, 2),
            "alu_achieved_Tops": round(achieved / 1e12, 3),
            "alu_peak_Tops": round(VALU_PEAK_LANE_OPS / 1e12, 2),
            "alu_frac": round(achieved / VALU_PEAK_LANE_OPS, 4)}


# ------------------------------------------------------------- GPU timing --
def load_traffic(key: str, kernel: str):
    """HBM bytes per launch from the rocprofv3 counter runs, if they were
    taken on the current sources of `kernel` (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get(key)
    if not ent or ent.get("source_digest") != source_digest(kernel):
        return None
    return ent.get("bytes_per_launch")


# --------------------------------------------------------------- workloads --
class Headline:
    """Eight workers' INT8 (s = 127) + error-feedback quantize of 256M fp32
    elements each (bucket d = 512, Philox seed w, step t), then the W = 8
    dequantize-accumulate into one fp32 average (alpha = 1/8, beta = 0).

    The eight gradients (seeded, resident in HBM), residuals and payloads
    are 18.4 GB, so no launch finds its working set in the 256 MB last-level
    cache; each worker's residual is carried from step to step."""

    KEY = "int8_ef_d512_n256M"
    AGG_KEY = "int8_w8_n256M:aggregate"
    KERNEL = "k_stream_quant<0, 8, 128, 1>"      # its kernels in the counter runs
    AGG_KERNEL = "k_deq_acc_wide<0, 8, 8, true>"
    CPU_PREFIX = 1 << 25        # elements of each worker kept for the oracle

    def __init__(self, torch, gq, WL, stream):
        self.torch, self.gq, self.stream = torch, gq, stream
        self.W, self.n = WL.WORKERS_W, WL.WORKERS_N
        self.desc = gq.desc(gq.GQ_UNIFORM, 512, s=127)
        self.bits = gq.gq_code_bits(self.desc)
        t0 = time.time()
        self.G, self.E, self.C, self.M, self.host = [], [], [], [], []
        for w in range(1, self.W + 1):
            h = WL.worker_gradient(w)
            self.host.append(h[: self.CPU_PREFIX].copy())
            self.G.append(torch.from_numpy(h).cuda())
            del h
            self.E.append(torch.zeros(self.n, dtype=torch.float32, device="cuda"))
            c, m = gq.alloc_payload(self.desc, self.n)
            self.C.append(c)
            self.M.append(m)
        self.avg = torch.empty(self.n, dtype=torch.float32, device="cuda")
        log(f"headline: {self.W} x {self.n} worker inputs in {time.time() - t0:.1f}s")
        self.q = [gq.PreparedQuantize(self.desc, self.G[w], self.E[w], self.C[w],
                                      self.M[w], stream) for w in range(self.W)]
        self.dq = gq.PreparedDequantizeAccumulate(
            self.desc, self.n, self.C, self.M, 1.0 / self.W, 0.0, self.avg, stream)

    def step(self, t: int, ev=None):
        """One step; with ev (W + 2 events) an event is recorded on the
        launch stream before every launch and after the last."""
        for w in range(self.W):
            if ev is not None:
                ev[w].record(self.stream)
            self.q[w](w + 1, t)
        if ev is not None:
            ev[self.W].record(self.stream)
        self.dq()
        if ev is not None:
            ev[self.W + 1].record(self.stream)

    def qbytes(self):
        return quant_bytes(self.bits, 1, 512, self.n, True)

    def dbytes(self):
        return deq_bytes(self.bits, 1, 512, self.n, self.W, 0.0)

    def release(self):
        del self.q, self.dq, self.G, self.E, self.C, self.M, self.avg


class Ternary:
    """Ternary + error feedback over the 25.6M-element layered gradient,
    then dequantize (W = 1), cycling the five seeded steps.

    Two buffer sets (residual, payload, output) alternate between
    consecutive steps, so even and odd steps form two independent
    error-feedback chains: a residual is read two steps after it was
    written, with ~0.6 GB of other traffic in between, and a step's
    working set is not left in the 256 MB last-level cache by the step
    before it."""

    SEED = 2
    KEY = "ternary_ef_d512_n25.6M"
    SETS = 2

    def __init__(self, torch, gq, WL, stream):
        self.torch, self.gq, self.stream = torch, gq, stream
        self.n = WL.TERNARY_N
        self.host = [WL.ternary_gradient(t) for t in range(WL.TERNARY_STEPS)]
        self.G = [torch.from_numpy(h).cuda() for h in self.host]
        self.desc = gq.desc(gq.GQ_UNIFORM, 512, s=1)
        self.bits = gq.gq_code_bits(self.desc)
        self.E, self.codes, self.meta, self.out = [], [], [], []
        for _ in range(self.SETS):
            self.E.append(torch.zeros(self.n, dtype=torch.float32, device="cuda"))
            c, m = gq.alloc_payload(self.desc, self.n)
            self.codes.append(c)
            self.meta.append(m)
            self.out.append(torch.empty(self.n, dtype=torch.float32, device="cuda"))
        # q[t mod 10]: gradient t mod 5 with buffer set t mod 2
        self.q = [gq.PreparedQuantize(self.desc, self.G[t % len(self.G)],
                                      self.E[t % self.SETS],
                                      self.codes[t % self.SETS],
                                      self.meta[t % self.SETS], stream)
                  for t in range(len(self.G) * self.SETS)]
        self.dq = [gq.PreparedDequantizeAccumulate(
            self.desc, self.n, [self.codes[k]], [self.meta[k]], 1.0, 0.0,
            self.out[k], stream) for k in range(self.SETS)]

    def quantize(self, t: int):
        self.q[t % len(self.q)](self.SEED, t)

    def dequantize(self, t: int):
        self.dq[t % self.SETS]()

    def step(self, t: int):
        self.quantize(t)
        self.dequantize(t)

    def qbytes(self):
        return quant_bytes(self.bits, 1, 512, self.n, True)

    def dbytes(self):
        return deq_bytes(self.bits, 1, 512, self.n, 1, 0.0)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(hl: Headline, repeats: int = 3):
    """The oracle on the host, on a bounded sample of the headline step: the
    first 2^25 elements of each of the eight workers (whole buckets),
    quantized INT8 + error feedback from a zero residual (Philox seed w, step
    0, global element indices from 0), then their W = 8 average.  Best of
    `repeats` wall times with all the OpenMP threads the host gives the
    oracle, and again with one thread on the first 2^22 elements of each
    worker."""
    import numpy as np

    import oracle as O

    od = O.Desc(O.UNIFORM, 512, s=127)

    def run(m: int) -> float:
        best = float("inf")
        for _ in range(repeats):
            t0 = time.perf_counter()
            cs, ms_ = [], []
            for w in range(hl.W):
                g = hl.host[w][:m]
                c, mm, _, _ = O.quantize(od, g, np.zeros(m, np.float32),
                                         seed=w + 1, step=0)
                cs.append(c)
                ms_.append(mm)
            O.dequantize_accumulate(od, m, cs, ms_, 1.0 / hl.W, 0.0)
            best = min(best, time.perf_counter() - t0)
        return best

    th = O.threads()
    m_all = hl.CPU_PREFIX
    t_all = run(m_all)
    O.set_threads(1)
    try:
        m_one = 1 << 22
        t_one = run(m_one)
    finally:
        O.set_threads(th)
    gbs = lambda m, t: round(4 * m * hl.W / t / 1e9, 4)  # noqa: E731
    return {"value": gbs(m_all, t_all), "unit": "GB/s", "cores": th,
            "kind": "oracle",
            "sample": (f"the headline step on the first {m_all} elements of "
                       f"each of {hl.W} workers: INT8 + EF quantize, then the "
                       f"W={hl.W} average; best of {repeats}: {t_all:.3f} s "
                       f"wall on {th} OpenMP threads"),
            "t1_value": gbs(m_one, t_one),
            "t1_sample": (f"same step on the first {m_one} elements of each "
                          f"worker, one thread, best of {repeats}: "
                          f"{t_one:.3f} s"),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


_LAST_TIMING = {}


def _stats(durs):
    """Median, mean, 10th / 90th percentile and count of per-launch times."""
    s = sorted(durs)
    q = lambda f: s[min(len(s) - 1, int(f * (len(s) - 1) + 0.5))]  # noqa: E731
    return {"median": q(0.5), "mean": sum(s) / len(s), "p10": q(0.1),
            "p90": q(0.9), "runs": len(s)}


def time_launches(torch, stream, launch, reps: int, warm: int = 3,
                  min_sample_ms: float = 0.5) -> dict:
    """Per-launch durations from `reps` samples on the launch stream: each
    sample is a batch of B back-to-back launches between two HIP events,
    B chosen so a sample lasts at least `min_sample_ms` (1 for launches of
    that length and more), and its per-launch time the batch time / B.  An
    event pair around every short launch would add the event's own
    dispatch (~4-5 us) to each; back to back, the samples carry only the
    gaps between consecutive kernels."""
    for i in range(warm):
        launch(i)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    launch(warm)
    b.record(stream)
    b.synchronize()
    est = a.elapsed_time(b)
    B = max(1, min(256, int(math.ceil(min_sample_ms / max(est, 1e-4)))))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    k = warm + 1
    ev[0].record(stream)
    for r in range(reps):
        for _ in range(B):
            launch(k)
            k += 1
        ev[r + 1].record(stream)
    ev[-1].synchronize()
    st = _stats([ev[r].elapsed_time(ev[r + 1]) / B for r in range(reps)])
    st["batch"] = B
    _LAST_TIMING["stats"] = st
    return st


def time_back_to_back(torch, stream, launch, reps: int, warm: int = 3) -> float:
    """Median per-launch duration in ms (see time_launches)."""
    return time_launches(torch, stream, launch, reps, warm)["median"]


def copy_reference(torch, stream, nbytes: int = 1 << 30) -> dict:
    """A plain read-once / write-once pass of known size (torch's negation,
    128-bit vectorised): what a streaming kernel reaches on this GPU."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    src.normal_()
    dst = torch.empty_like(src)
    ms = time_back_to_back(torch, stream,
                           lambda i: torch.neg(src, out=dst), 20)
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    return {"kernel": f"reference copy (read {nbytes >> 20} MiB + write)",
            "ms": round(ms, 5), "moved_GBps": round(gbs, 2),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm"}


def time_oracle(run, size: int, d: int, budget: float = 0.5,
                max_n: int = 1 << 22):
    """Throughput (GB/s of fp32 input) of run(n), a CPU oracle call on the
    first n elements (whole buckets of d), n growing until `budget` seconds."""
    import oracle as O

    n = min(size, 1 << 16)
    n -= n % d if n > d else 0
    while True:
        t0 = time.perf_counter()
        run(n)
        dt = time.perf_counter() - t0
        if dt >= budget or n >= min(max_n, size):
            return {"oracle_GBps": round(4 * n / dt / 1e9, 4),
                    "oracle_elements": n, "oracle_threads": O.threads()}
        n = min(4 * n, max_n, size)


# Oracle timings wait here until every GPU measurement is done: the oracle's
# OpenMP threads, run between two GPU timings, slowed the next GPU kernel by
# up to 8 % (INT8 W = 8 dequantize-accumulate: 514 -> 557 us).
DEFERRED = []


def oracle_rate(host_g, desc_kw, ef: bool, seed: int = 0, budget: float = 0.5,
                max_n: int = 1 << 22):
    """The CPU oracle's quantize throughput on a prefix of the same input,
    measured later by run_deferred() (entry() registers the job)."""
    import numpy as np

    import oracle as O

    od = O.Desc(**desc_kw)
    host_g = host_g[:max_n].copy()

    def run(n):
        e = np.zeros(n, dtype=np.float32) if ef else None
        O.quantize(od, host_g[:n], e, seed=seed, step=0)
    return {"_oracle": lambda: time_oracle(run, host_g.size, od.d, budget,
                                           max_n)}


def run_deferred() -> None:
    """Runs the oracle timings entry() queued and fills in their entries."""
    for r, job in DEFERRED:
        r.update(job())
    DEFERRED.clear()


def entry(name, ms, nbytes, n, bound="hbm", extra=None, alu=None):
    """One kernel's line: `ms` is the median per-launch duration of the
    timing just taken (its spread is attached), `alu` the algorithmic
    lane-operations per element of an ALU-bound kernel."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    r = {"kernel": name, "ms": round(ms, 5),
         "elements_per_s": round(n / (ms * 1e-3)),
         "logical_GBps": round(4 * n / (ms * 1e-3) / 1e9, 2),
         "moved_GBps": round(gbs, 2), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
         "bound": bound}
    st = _LAST_TIMING.pop("stats", None)
    if st is not None and st["median"] == ms:
        r.update({"ms_mean": round(st["mean"], 5), "ms_p10": round(st["p10"], 5),
                  "ms_p90": round(st["p90"], 5), "runs": st["runs"],
                  "launches_per_run": st.get("batch", 1)})
    if alu is not None:
        r.update(alu_fields(alu, n, ms))
    if extra:
        r.update(extra)
        job = r.pop("_oracle", None)
        if job is not None:
            DEFERRED.append((r, job))
    return r


def suite(torch, gq, WL, stream, reps: int, only: str | None = None):
    """Every other workload's kernels, each timed back to back (only the
    workloads whose name contains `only`: qsgd, orq, bingrad, ternary,
    dense, nearest, layers, topk, elias)."""
    out = []
    tb = lambda f, r=reps: time_back_to_back(torch, stream, f, r)  # noqa: E731
    want = lambda name: only is None or only in name  # noqa: E731

    suites = [("qsgd", lambda: suite_qsgd(torch, gq, WL, stream, tb)),
              ("orq", lambda: suite_orq(torch, gq, WL, stream, tb, reps)),
              ("bingrad", lambda: suite_bingrad(torch, gq, WL, stream, tb, reps)),
              ("ternary", lambda: suite_ternary(torch, gq, WL, stream, tb, reps)),
              ("dense", lambda: suite_dense(torch, gq, WL, stream, tb, reps)),
              ("nearest", lambda: suite_nearest(torch, gq, WL, stream, tb, reps)),
              ("layers", lambda: suite_layers(torch, gq, WL, stream, tb)),
              ("topk", lambda: suite_topk(torch, gq, WL, stream, tb)),
              ("elias", lambda: suite_elias(torch, gq, WL, stream, tb))]
    for name, run in suites:
        if want(name):
            out += run()
            # each workload starts from memory handed back to the driver: a
            # suite placed in the 18 GB the headline's buffers left cached ran up
            # to 20 % slower than alone
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    return out


def suite_elias(torch, gq, WL, stream, tb):
    """Elias gamma coding of the 25.6M layered gradient's codes (d = 512),
    QSGD s = 4 and ternary s = 1: encode (count, scan and record passes) and
    decode, two alternating payloads.  Moved bytes: encode reads the codes
    twice and writes the stream and the offsets; decode reads the stream and
    offsets and writes the codes."""
    import numpy as np

    import oracle as O
    out = []
    hosts = [WL.ternary_gradient(0), WL.ternary_gradient(1)]
    G = [torch.from_numpy(h).cuda() for h in hosts]
    n = G[0].numel()
    for s in (4, 1):
        d = gq.desc(gq.GQ_UNIFORM, 512, s=s)
        cb, cap, mf = gq.gq_payload_size(d, n)
        P = [gq.alloc_payload(d, n) for _ in range(2)]
        for k in range(2):
            gq.gq_quantize(d, G[k], None, 2, k, P[k][0], P[k][1], stream)
        S = [gq.alloc_elias(d, n) for _ in range(2)]
        back = [torch.empty(cap, dtype=torch.uint8, device="cuda") for _ in range(2)]
        ms = tb(lambda i: gq.gq_elias_encode(d, n, P[i % 2][0], S[i % 2][0],
                                             S[i % 2][1], stream))
        torch.cuda.synchronize()
        nb = S[0][0].numel() - 1
        nw = int(S[0][0][-1].item())
        codes_h = P[0][0][:cb].cpu().numpy()
        oracle = {"_oracle": lambda s_=s, ch=codes_h: time_oracle(
            lambda k: O.elias_encode(512, s_, k, ch), n, 512)}
        stream_bytes = 4 * nw + 8 * (nb + 1)
        extra = {"bits_per_element": round(32 * nw / n, 4),
                 "fixed_bits": 8 * cb / n,
                 "compression_vs_fp32": round(4 * n / (stream_bytes + 4 * mf), 3),
                 "compression_fixed": round(4 * n / (cb + 4 * mf), 3)}
        out.append(entry(f"elias encode s={s} d=512 n={n}", ms,
                         2 * cb + 4 * nw + 3 * 8 * nb, n, bound="alu",
                         extra={**extra, **oracle}, alu=elias_encode_ops()))
        ms = tb(lambda i: gq.gq_elias_decode(d, n, S[i % 2][0], S[i % 2][1],
                                             back[i % 2], stream=stream))
        out.append(entry(f"elias decode s={s} d=512 n={n}", ms,
                         4 * nw + 8 * (nb + 1) + cb, n, bound="latency"))
        torch.cuda.synchronize()
        assert torch.equal(back[0][:cb], P[0][0][:cb])
        del P, S, back
    return out


def suite_topk(torch, gq, WL, stream, tb):
    """Top-K with quantization: the 25.6M layered gradient, K = 26 of every
    512 (about 5 %), 4-bit values (s = 4), error feedback; and its
    dequantize."""
    import numpy as np

    import oracle as O
    out = []
    host = WL.ternary_gradient(0)
    G = [torch.from_numpy(host).cuda(),
         torch.from_numpy(WL.ternary_gradient(1)).cuda()]
    n = G[0].numel()
    E = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    d = gq.desc(gq.GQ_TOPK, 512, s=4, levels=26)
    cb, _, mf = gq.gq_payload_size(d, n)
    P = [gq.alloc_payload(d, n) for _ in range(2)]
    O_ = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    qs = [gq.PreparedQuantize(d, G[k], E[k], P[k][0], P[k][1], stream) for k in range(2)]
    ms = tb(lambda i: qs[i % 2](2, i))
    oracle = {"_oracle": lambda: time_oracle(
        lambda k: O.quantize_topk(512, 4, 26, host[:k], np.zeros(k, np.float32),
                                  seed=2), n, 512)}
    out.append(entry(f"quantize top-k 26/512 s=4 +ef n={n}", ms,
                     12 * n + cb + 4 * mf, n, bound="alu", alu=topk_ops(512, 26),
                     extra={"compression_vs_fp32": round(4 * n / (cb + 4 * mf), 3),
                            **oracle}))
    dqs = [gq.PreparedDequantizeAccumulate(d, n, [P[k][0]], [P[k][1]], 1.0, 0.0,
                                           O_[k], stream) for k in range(2)]
    ms = tb(lambda i: dqs[i % 2]())
    out.append(entry(f"dequantize top-k 26/512 W=1 n={n}", ms, cb + 4 * mf + 4 * n, n))
    return out


def suite_layers(torch, gq, WL, stream, tb):
    """Per-layer scale (TernGrad): ternary + EF on the 25.6M gradient with
    one scale for each of its 160 layers, and its dequantize.  The quantizer
    makes two passes (layer maxima, then rounding): 8 + 12 bytes per element
    plus codes and scales."""
    import numpy as np
    out = []
    import oracle as O
    sizes, _ = WL.ternary_layout()
    off_h = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    off = torch.from_numpy(off_h).cuda()
    nl = len(sizes)
    host = WL.ternary_gradient(0)
    G = [torch.from_numpy(host).cuda(),
         torch.from_numpy(WL.ternary_gradient(1)).cuda()]
    n = G[0].numel()
    E = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    d = gq.desc(gq.GQ_UNIFORM, 512, s=1)
    _, cap, _ = gq.gq_payload_size(d, n)
    C = [torch.empty(cap, dtype=torch.uint8, device="cuda") for _ in range(2)]
    M = [torch.empty(nl, dtype=torch.float32, device="cuda") for _ in range(2)]
    O_ = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    ms = tb(lambda i: gq.gq_quantize_layers(d, off, G[i % 2], E[i % 2], 2, i,
                                            C[i % 2], M[i % 2], stream))
    def oracle_layers(k):
        o = [int(x) for x in off_h if x < k] + [k]
        O.quantize_layers(O.Desc(O.UNIFORM, s=1), o, host[:k],
                          np.zeros(k, np.float32), seed=2)
    out.append(entry(f"quantize ternary+ef per-layer scale ({nl} layers) n={n}",
                     ms, 20 * n + (2 * n + 7) // 8 + 4 * nl, n,
                     extra={"_oracle": lambda: time_oracle(oracle_layers, n, 512)}))
    ms = tb(lambda i: gq.gq_dequantize_accumulate_layers(
        d, n, off, [C[i % 2]], [M[i % 2]], 1.0, 0.0, O_[i % 2], stream))
    out.append(entry(f"dequantize ternary per-layer scale W=1 n={n}", ms,
                     (2 * n + 7) // 8 + 4 * nl + 4 * n, n))
    # layer-wise bit allocation over the same layers and their scales: one
    # block, latency-bound (reads offsets and scales, writes widths and
    # segment offsets)
    Wd = torch.empty(nl, dtype=torch.int32, device="cuda")
    Sg = torch.empty(nl + 1, dtype=torch.int64, device="cuda")
    ms = tb(lambda i: gq.gq_allocate_layer_bits(n, off, M[0], 3 * n, Wd, Sg, stream))
    out.append(entry(f"allocate layer bits ({nl} layers, 3 bits per element)", ms,
                     8 * (nl + 1) + 4 * nl + 4 * nl + 8 * (nl + 1), nl,
                     bound="latency"))
    # the payload of that allocation: each layer at its own width (two
    # passes as above: 8 + 12 bytes per element, plus the mixed-width codes)
    gq.gq_allocate_layer_bits(n, off, M[0], 3 * n, Wd, Sg, stream)
    torch.cuda.synchronize()
    widths_h = Wd.cpu().numpy().tolist()
    pb = int(Sg[-1].item())
    cap_a = gq.gq_alloc_payload_bytes(n, nl)
    PA = [torch.empty(cap_a, dtype=torch.uint8, device="cuda") for _ in range(2)]
    ms = tb(lambda i: gq.gq_quantize_layers_alloc(off, G[i % 2], E[i % 2], Wd, Sg, 2,
                                                  i, PA[i % 2], M[i % 2],
                                                  stream=stream))

    def oracle_alloc(k):
        o = [int(x) for x in off_h if x < k] + [k]
        O.quantize_layers_alloc(o, host[:k], np.zeros(k, np.float32),
                                widths_h[:len(o) - 1], seed=2)
    wset = "/".join(str(b) for b in sorted(set(widths_h)))
    out.append(entry(f"quantize layer-wise widths {wset} ({nl} layers, "
                     f"{8 * pb / n:.2f} bits per element) +ef n={n}",
                     ms, 20 * n + pb + 4 * nl + 12 * nl, n,
                     extra={"_oracle": lambda: time_oracle(oracle_alloc, n, 512)}))
    ms = tb(lambda i: gq.gq_dequantize_accumulate_layers_alloc(
        n, off, [PA[i % 2]], [M[i % 2]], [Wd], [Sg], 1.0, 0.0, O_[i % 2], stream))
    out.append(entry(f"dequantize layer-wise widths W=1 n={n}", ms,
                     pb + 16 * nl + 4 * n, n))
    return out


def suite_nearest(torch, gq, WL, stream, tb, reps):
    """Deterministic rounding to the nearest level: ternary + EF on the
    25.6M layered gradient, ORQ-9 on 100M."""
    out = []
    N = gq.GQ_FLAG_NEAREST
    host = WL.ternary_gradient(0)
    g = torch.from_numpy(host).cuda()
    n = g.numel()
    e = torch.zeros_like(g)
    d = gq.desc(gq.GQ_UNIFORM, 512, s=1, flags=N)
    c, m = gq.alloc_payload(d, n)
    q = gq.PreparedQuantize(d, g, e, c, m, stream)
    ms = tb(lambda i: q(2, i))
    out.append(entry(f"quantize ternary+ef nearest d=512 n={n}", ms,
                     quant_bytes(2, 1, 512, n, True), n,
                     extra=oracle_rate(host, dict(scheme=0, d=512, s=1, flags=N),
                                       True, seed=2)))
    del g, e, c, m, q, host
    host = WL.orq_gradient()
    g = torch.from_numpy(host).cuda()
    n = g.numel()
    d = gq.desc(gq.GQ_ORQ, 512, levels=9, flags=N)
    c, m = gq.alloc_payload(d, n)
    q = gq.PreparedQuantize(d, g, None, c, m, stream)
    ms = tb(lambda i: q(3, 0), max(3, reps // 2))
    out.append(entry(f"quantize orq L=9 nearest d=512 n={n}", ms,
                     quant_bytes(4, 9, 512, n, False), n, bound="alu",
                     alu=orq_ops(9, 512),
                     extra=oracle_rate(host, dict(scheme=3, d=512, L=9, flags=N),
                                       False, seed=3)))
    return out


def suite_dense(torch, gq, WL, stream, tb, reps):
    """Dense packing (8 codes per base-A field): ternary + EF on the 25.6M
    layered gradient and its dequantize, ORQ-3 / ORQ-9 on 100M."""
    out = []
    D = gq.GQ_FLAG_DENSE

    def ratio(d, n):
        cb, _, mf = gq.gq_payload_size(d, n)
        return {"compression_vs_fp32": round(4 * n / (cb + 4 * mf), 3),
                "code_bytes": cb}

    host = WL.ternary_gradient(0)
    g = torch.from_numpy(host).cuda()
    n = g.numel()
    e = torch.zeros_like(g)
    d = gq.desc(gq.GQ_UNIFORM, 512, s=1, flags=D)
    c, m = gq.alloc_payload(d, n)
    q = gq.PreparedQuantize(d, g, e, c, m, stream)
    ms = tb(lambda i: q(2, i))
    cb = ratio(d, n)
    out.append(entry(f"quantize ternary+ef dense d=512 n={n}", ms,
                     12 * n + cb["code_bytes"] + 4 * ((n + 511) // 512), n,
                     extra={**cb, **oracle_rate(host, dict(scheme=0, d=512, s=1,
                                                           flags=2), True, seed=2)}))
    o = torch.empty_like(g)
    dq = gq.PreparedDequantizeAccumulate(d, n, [c], [m], 1.0, 0.0, o, stream)
    ms = tb(lambda i: dq())
    out.append(entry(f"dequantize ternary dense W=1 n={n}", ms,
                     cb["code_bytes"] + 4 * ((n + 511) // 512) + 4 * n, n))
    del g, e, c, m, q, o, dq, host

    host = WL.orq_gradient()
    g = torch.from_numpy(host).cuda()
    n = g.numel()
    for L in (3, 9):
        d = gq.desc(gq.GQ_ORQ, 512, levels=L, flags=D)
        c, m = gq.alloc_payload(d, n)
        q = gq.PreparedQuantize(d, g, None, c, m, stream)
        ms = tb(lambda i: q(3, 0), max(3, reps // 2))
        cb = ratio(d, n)
        out.append(entry(f"quantize orq L={L} dense d=512 n={n}", ms,
                         4 * n + cb["code_bytes"] + 4 * L * ((n + 511) // 512),
                         n, bound="alu", alu=orq_ops(L, 512),
                         extra={**cb, **oracle_rate(host, dict(scheme=3, d=512,
                                                               L=L, flags=2),
                                                    False, seed=3)}))
        del c, m, q
    return out


def suite_qsgd(torch, gq, WL, stream, tb):
    """QSGD s=4, 65,536 elements: cache-resident, latency-bound."""
    out = []
    host = WL.qsgd_gradient()
    g = torch.from_numpy(host).cuda()
    d = gq.desc(gq.GQ_UNIFORM, 512, s=4)
    c, m = gq.alloc_payload(d, g.numel())
    o = torch.empty_like(g)
    q = gq.PreparedQuantize(d, g, None, c, m, stream)
    ms = tb(lambda i: q(0, 0))
    out.append(entry("quantize qsgd s=4 d=512 n=65536", ms,
                     quant_bytes(4, 1, 512, g.numel(), False), g.numel(),
                     bound="latency",
                     extra=oracle_rate(host, dict(scheme=0, d=512, s=4), False)))
    dq = gq.PreparedDequantizeAccumulate(d, g.numel(), [c], [m], 1.0, 0.0, o,
                                         stream)
    ms = tb(lambda i: dq())
    out.append(entry("dequantize qsgd W=1 n=65536", ms,
                     deq_bytes(4, 1, 512, g.numel(), 1, 0.0), g.numel(),
                     bound="latency"))
    del g, c, m, o, q, dq
    # supplementary: the same recipe and shape at n = 2^28 (the stream's first
    # 65,536 values are the workload above), where the uniform no-EF path is
    # HBM-bound rather than launch-bound
    n = 1 << 28
    g = torch.from_numpy(WL.qsgd_gradient(n)).cuda()
    c, m = gq.alloc_payload(d, n)
    o = torch.empty_like(g)
    q = gq.PreparedQuantize(d, g, None, c, m, stream)
    ms = tb(lambda i: q(0, 0))
    out.append(entry(f"quantize qsgd s=4 d=512 n={n} (supplementary)", ms,
                     quant_bytes(4, 1, 512, n, False), n))
    dq = gq.PreparedDequantizeAccumulate(d, n, [c], [m], 1.0, 0.0, o, stream)
    ms = tb(lambda i: dq())
    out.append(entry(f"dequantize qsgd W=1 n={n} (supplementary)", ms,
                     deq_bytes(4, 1, 512, n, 1, 0.0), n))
    return out


def orq_attach_traffic(ent: dict, L: int, bisect: bool, algorithmic: int) -> None:
    tr = load_traffic(orq_traffic_key(L, bisect), "orq")
    ent["traffic"] = tr
    if tr:
        ent["traffic_ratio"] = round(tr / algorithmic, 4)


def suite_orq(torch, gq, WL, stream, tb, reps):
    """ORQ-5 / ORQ-9 on 100M elements, clip off / on."""
    out = []
    t0 = time.time()
    host = WL.orq_gradient()
    g = torch.from_numpy(host).cuda()
    log(f"suite: orq input in {time.time() - t0:.1f}s")
    n = g.numel()
    for L in (5, 9):
        for clip in (0, 1):
            d = gq.desc(gq.GQ_ORQ, 512, levels=L, flags=clip, clip_sigma=3.0)
            c, m = gq.alloc_payload(d, n)
            bits = gq.gq_code_bits(d)
            q = gq.PreparedQuantize(d, g, None, c, m, stream)
            ms = tb(lambda i: q(3, 0), max(3, reps // 2))
            out.append(entry(f"quantize orq L={L} clip={clip} d=512 n={n}", ms,
                             quant_bytes(bits, L, 512, n, False), n,
                             bound="alu", alu=orq_ops(L, 512, clip=bool(clip)),
                             extra=oracle_rate(
                                 host, dict(scheme=3, d=512, L=L, flags=clip,
                                            clip_sigma=3.0), False, seed=3)))
            orq_attach_traffic(out[-1], L, False, quant_bytes(bits, L, 512, n, False))
            del c, m, q
    # the recursive-bisection reading of the level selection
    for L in (5, 9):
        d = gq.desc(gq.GQ_ORQ, 512, levels=L, flags=gq.GQ_FLAG_BISECT)
        c, m = gq.alloc_payload(d, n)
        q = gq.PreparedQuantize(d, g, None, c, m, stream)
        ms = tb(lambda i: q(3, 0), max(3, reps // 2))
        out.append(entry(f"quantize orq L={L} bisect d=512 n={n}", ms,
                         quant_bytes(gq.gq_code_bits(d), L, 512, n, False), n,
                         bound="alu", alu=orq_ops(L, 512, bisect=True),
                         extra=oracle_rate(
                             host, dict(scheme=3, d=512, L=L, flags=8), False,
                             seed=3)))
        orq_attach_traffic(out[-1], L, True,
                           quant_bytes(gq.gq_code_bits(d), L, 512, n, False))
        del c, m, q
    return out


def suite_bingrad(torch, gq, WL, stream, tb, reps):
    """BinGrad-b (optimal two-level), the sign split and the min/max two-level
    quantizer with error feedback, 1B elements, over the bucket sweep."""
    out = []
    t0 = time.time()
    host = WL.bingrad_gradient()
    g = torch.from_numpy(host).cuda()
    log(f"suite: bingrad input in {time.time() - t0:.1f}s")
    n = g.numel()
    e = torch.zeros_like(g)
    for scheme, nm in ((gq.GQ_BIN_OPT, "bin_opt"), (gq.GQ_BIN_SIGN, "bin_sign")):
        for dd in BINGRAD_BUCKETS:
            d = gq.desc(scheme, dd)
            c, m = gq.alloc_payload(d, n)
            e.zero_()
            q = gq.PreparedQuantize(d, g, e, c, m, stream)
            ms = tb(lambda i: q(0, i), max(3, reps // 2))
            out.append(entry(f"quantize {nm}+ef d={dd} n={n}", ms,
                             quant_bytes(1, 2, dd, n, True), n,
                             bound="alu" if scheme == gq.GQ_BIN_OPT else "hbm",
                             alu=(None if scheme != gq.GQ_BIN_OPT else
                                  binopt_prune_ops() if dd >= 1024 else binopt_ops(dd)),
                             extra=oracle_rate(host, dict(scheme=scheme, d=dd),
                                               True)))
            if scheme == gq.GQ_BIN_OPT:
                tr = load_traffic(f"bin_opt_ef_d{dd}_n1B", "bin_opt")
                out[-1]["traffic"] = tr
                if tr:
                    out[-1]["traffic_ratio"] = round(
                        tr / quant_bytes(1, 2, dd, n, True), 4)
            del c, m, q
    # the min/max two-level quantizer (ORQ with L = 2, read as BinGrad-pb)
    for dd in (128, 512, 2048, 8192, 32768):
        d = gq.desc(gq.GQ_ORQ, dd, levels=2)
        c, m = gq.alloc_payload(d, n)
        e.zero_()
        q = gq.PreparedQuantize(d, g, e, c, m, stream)
        ms = tb(lambda i: q(0, i), max(3, reps // 2))
        out.append(entry(f"quantize bin_pb (orq L=2)+ef d={dd} n={n}", ms,
                         quant_bytes(1, 2, dd, n, True), n,
                         extra=oracle_rate(host, dict(scheme=3, d=dd, L=2), True)))
        del c, m, q
    return out


def suite_ternary(torch, gq, WL, stream, tb, reps):
    """Ternary (s = 1, 2-bit) + error feedback on the 25.6M layered gradient
    (160 Laplace layers, d = 512), quantize and dequantize W = 1, with two
    alternating buffer sets so no launch finds its data in the last-level
    cache; and the whole step (quantize + dequantize) back to back."""
    tw = Ternary(torch, gq, WL, stream)
    out = []
    ms = tb(tw.quantize, max(20, reps))
    out.append(entry(f"quantize ternary+ef d=512 n={tw.n}", ms, tw.qbytes(),
                     tw.n, extra=oracle_rate(tw.host[0], dict(scheme=0, d=512, s=1),
                                             True, seed=2)))
    ms = tb(tw.dequantize, max(20, reps))
    out.append(entry(f"dequantize ternary W=1 n={tw.n}", ms, tw.dbytes(), tw.n))
    ms = tb(tw.step, max(20, reps))
    out.append(entry(f"step ternary+ef quantize + dequantize n={tw.n}", ms,
                     tw.qbytes() + tw.dbytes(), tw.n))
    return out


# ------------------------------------------------------- counter ingestion --
def ingest(dirs):
    """Combine two rocprofv3 --pmc runs of `bench.py --counters` (one with
    FETCH_SIZE, one with WRITE_SIZE; rocpd databases) into
    profiles/traffic.json.  Each counter is scaled by what it reads for the
    known-size negation pass in the same run (COPY_BYTES read, COPY_BYTES
    written), and each kernel's value is the median over its dispatches."""
    import sqlite3

    vals = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
            con = sqlite3.connect(path)
            for name, cn, v in con.execute(
                    "select kernel_name, counter_name, value "
                    "from counters_collection"):
                vals.setdefault((cn, name), []).append(float(v))
            con.close()

    def med(cn, pred):
        for (c, name), v in vals.items():
            if c == cn and pred(name):
                v = sorted(v)
                return name, v[len(v) // 2]
        raise KeyError(f"{cn}: kernel not found in the counter runs")

    is_copy = lambda k: "neg_kernel" in k  # noqa: E731
    f_scale = COPY_BYTES / (med("FETCH_SIZE", is_copy)[1] * 1024.0)
    w_scale = COPY_BYTES / (med("WRITE_SIZE", is_copy)[1] * 1024.0)
    res = {"_calibration": {
        "copy_bytes": COPY_BYTES, "fetch_scale": round(f_scale, 5),
        "write_scale": round(w_scale, 5),
        "note": ("counters are KiB per dispatch; traffic = FETCH_SIZE*1024*"
                 "fetch_scale + WRITE_SIZE*1024*write_scale")}}
    for key, tag, sig in ((Headline.KEY, "k_stream_quant", Headline.KERNEL),
                          (Headline.AGG_KEY, "k_deq_acc", Headline.AGG_KERNEL)):
        kname, f = med("FETCH_SIZE", lambda k, t=sig: t in k)
        _, w = med("WRITE_SIZE", lambda k, t=sig: t in k)
        res[key] = {"kernel": kname, "source_digest": source_digest(tag),
                    "fetch_kib": f, "write_kib": w,
                    "bytes_per_launch": round(f * 1024 * f_scale +
                                              w * 1024 * w_scale)}
    # BinGrad-b + EF on 1B (from `--counters --only bingrad`): a quantize
    # launch is the sort kernel (d <= 512) or the sort-free kernel plus the
    # sort kernel's pass over the buckets it left (d >= 1024); the whole-
    # bucket launches (the one-block launch of a short last bucket, when
    # there is one, is left out: under 1e-5 of the bytes)
    for dd in BINGRAD_BUCKETS:
        sigs = (f"k_wave_sort_quant<2, 1, {dd}, false, true>", f"k_sort_quant<2, 1, {dd}>",
                f"k_binopt_block<{dd}, true, true>")
        names, fk, wk = [], 0.0, 0.0
        for sig in sigs:
            try:
                kname, f = med("FETCH_SIZE", lambda k, t=sig: t in k)
                _, w = med("WRITE_SIZE", lambda k, t=sig: t in k)
            except KeyError:
                continue
            names.append(kname)
            fk, wk = fk + f, wk + w
        if names:
            res[f"bin_opt_ef_d{dd}_n1B"] = {
                "kernel": " + ".join(names), "source_digest": source_digest("bin_opt"),
                "fetch_kib": fk, "write_kib": wk,
                "bytes_per_launch": round(fk * 1024 * f_scale + wk * 1024 * w_scale)}
    # ORQ on 100M, d = 512 (from `--counters --only orq`): one kernel per
    # (L, bisection); clip on and off share it and move the same bytes
    for L, bis in ORQ_TRAFFIC:
        sig = f"k_wave_sort_quant<3, {3 if L == 5 else 4}, 512, {'true' if bis else 'false'}, true>"
        try:
            kname, f = med("FETCH_SIZE", lambda k, t=sig: t in k)
            _, w = med("WRITE_SIZE", lambda k, t=sig: t in k)
        except KeyError:
            continue
        res[orq_traffic_key(L, bis)] = {
            "kernel": kname, "source_digest": source_digest("orq"),
            "fetch_kib": f, "write_kib": w,
            "bytes_per_launch": round(f * 1024 * f_scale + w * 1024 * w_scale)}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res, indent=1))


# -------------------------------------------------------------------- main --
DIGEST_FILE = os.path.join(ROOT, "tests", "golden", "workload_digests.json")
CPU_CONFIGS_FILE = os.path.join(ROOT, "profiles", "cpu_oracle_configs.json")


def check_inputs(WL, named) -> dict:
    """numpy's version and whether the first 2^24-element chunk of each named
    input (name -> array, or list of arrays) hashes to its recorded digest."""
    import numpy as np
    try:
        with open(DIGEST_FILE) as f:
            ref = json.load(f)
    except (OSError, ValueError):
        return {"numpy": np.__version__, "digests": None}
    ok = {}
    for name, (arr, pick) in named.items():
        ok[name] = WL.chunk_sha256(arr[:WL.CHUNK])[0] == pick(ref)[0]
    return {"numpy": np.__version__, "digests_numpy": ref.get("numpy"),
            "first_chunk_sha256_match": ok,
            "digests": os.path.relpath(DIGEST_FILE, ROOT)}


def load_cpu_configs():
    """The oracle's rates at the workloads' full sizes (`bench.py
    --cpu-configs`, taken on the GPU machine's host), or None."""
    try:
        with open(CPU_CONFIGS_FILE) as f:
            return json.load(f)
    except (OSError, ValueError):
        return None


def cpu_configs() -> dict:
    """The CPU oracle on every workload at its full size (no prefix), on this
    host: all the OpenMP threads it gives the oracle and one thread.  Best
    of 3 for QSGD, ternary and ORQ, one run for BinGrad-b / sign split on 1B
    (two EF steps; one thread: step 0 at d = 512 only) and for the eight
    INT8 + EF workers and their average (all threads only).  Times exclude
    drawing the inputs.  Throughput = 4 bytes per input element per second
    (every element of every step or worker; the aggregation's inputs are
    counted once, with the quantizes)."""
    import numpy as np

    import oracle as O
    from communication_efficient_gradient_amd import workloads as WL

    th = O.threads()
    res = {"cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
           "threads": th, "numpy": np.__version__, "configs": []}

    def best(fn, reps):
        b = float("inf")
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            b = min(b, time.perf_counter() - t0)
        return b

    def add(name, n, fn, reps, one_reps):
        t = best(fn, reps)
        rec = {"config": name, "elements": n, "threads": th, "runs": reps,
               "s": round(t, 4), "elements_per_s": round(n / t),
               "GBps": round(4 * n / t / 1e9, 4)}
        if one_reps:
            O.set_threads(1)
            try:
                t1 = best(fn, one_reps)
            finally:
                O.set_threads(th)
            rec.update({"t1_runs": one_reps, "t1_s": round(t1, 4),
                        "t1_GBps": round(4 * n / t1 / 1e9, 4)})
        res["configs"].append(rec)
        log(f"cpu config: {rec}")

    # C1 QSGD s=4, 65,536, quantize + dequantize
    g = WL.qsgd_gradient()
    d1 = O.Desc(O.UNIFORM, 512, s=4)

    def c1():
        c, m, _, _ = O.quantize(d1, g, None, seed=0, step=0)
        O.dequantize_accumulate(d1, g.size, [c], [m], 1.0, 0.0)
    add("qsgd s=4 d=512 n=65536, quantize + dequantize", g.size, c1, 3, 3)
    # C2 ternary + EF, 5 steps over the 160-layer 25.6M gradient
    steps = [WL.ternary_gradient(t) for t in range(WL.TERNARY_STEPS)]
    d2 = O.Desc(O.UNIFORM, 512, s=1)

    def c2():
        e = np.zeros(WL.TERNARY_N, np.float32)
        for t, gt in enumerate(steps):
            c, m, e, _ = O.quantize(d2, gt, e, seed=2, step=t)
            O.dequantize_accumulate(d2, gt.size, [c], [m], 1.0, 0.0)
    add("ternary + EF d=512 n=25600000, 5 steps of quantize + dequantize",
        WL.TERNARY_N * WL.TERNARY_STEPS, c2, 3, 3)
    del steps
    # C3 ORQ-5 / ORQ-9, clip off / on, 100M
    g = WL.orq_gradient()
    for L in (5, 9):
        for clip in (0, 1):
            d3 = O.Desc(O.ORQ, 512, L=L, flags=clip, clip_sigma=3.0)
            add(f"orq L={L} clip={clip} d=512 n={g.size}", g.size,
                lambda d3=d3: O.quantize(d3, g, None, seed=3, step=0), 3, 3)
    del g
    # C4 BinGrad-b / sign split + EF, 1B, two steps
    g = WL.bingrad_gradient()
    for scheme, nm in ((O.BIN_OPT, "bin_opt"), (O.BIN_SIGN, "bin_sign")):
        for dd in BINGRAD_BUCKETS:
            d4 = O.Desc(scheme, dd)

            def c4(d4=d4):
                e = np.zeros(g.size, np.float32)
                for t in range(2):
                    _, _, e, _ = O.quantize(d4, g, e, seed=0, step=t)
            add(f"{nm} + EF d={dd} n={g.size}, steps 0 and 1", 2 * g.size, c4, 1, 0)
        d4 = O.Desc(scheme, 512)
        O.set_threads(1)
        try:
            t1 = best(lambda: O.quantize(d4, g, np.zeros(g.size, np.float32),
                                         seed=0, step=0), 1)
        finally:
            O.set_threads(th)
        rec = next(r for r in res["configs"]
                   if r["config"].startswith(f"{nm} + EF d=512 "))
        rec.update({"t1_runs": 1, "t1_s": round(t1, 4), "t1_config": "step 0 only",
                    "t1_GBps": round(4 * g.size / t1 / 1e9, 4)})
        log(f"cpu config: {rec}")
    del g
    # C5 eight INT8 + EF workers of 256M and their W = 8 average
    d5 = O.Desc(O.UNIFORM, 512, s=127)
    gs = [WL.worker_gradient(w) for w in range(1, WL.WORKERS_W + 1)]

    def c5():
        cs, ms_ = [], []
        for w, gw in enumerate(gs, start=1):
            c, m, _, _ = O.quantize(d5, gw, np.zeros(gw.size, np.float32),
                                    seed=w, step=0)
            cs.append(c)
            ms_.append(m)
        O.dequantize_accumulate(d5, WL.WORKERS_N, cs, ms_, 1.0 / WL.WORKERS_W, 0.0)
    add(f"int8 + EF d=512, {WL.WORKERS_W} workers x {WL.WORKERS_N}, then the "
        f"W={WL.WORKERS_W} average", WL.WORKERS_W * WL.WORKERS_N, c5, 1, 0)
    return res


def load_parity():
    """Whole-payload parity counts of the full-size workloads, as the GPU
    tests last recorded them (tie buckets and mismatched elements per
    configuration), or None."""
    try:
        with open(PARITY_FILE) as f:
            return json.load(f)
    except (OSError, ValueError):
        return None


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--suite", choices=("main", "all"), default="all")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--only", choices=("qsgd", "orq", "bingrad", "ternary",
                                       "dense", "nearest", "layers", "topk",
                                       "elias"),
                    help="time only this workload's kernels after the headline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="short run for rocprofv3 --pmc: headline steps + a copy")
    ap.add_argument("--ingest", nargs="+", metavar="DIR")
    ap.add_argument("--cpu-configs", action="store_true",
                    help="time the CPU oracle on every workload at its full "
                         "size and store the result in profiles/ (no GPU)")
    args = ap.parse_args()

    if args.ingest:
        ingest(args.ingest)
        return 0
    if args.cpu_configs:
        res = cpu_configs()
        os.makedirs(os.path.dirname(CPU_CONFIGS_FILE), exist_ok=True)
        with open(CPU_CONFIGS_FILE, "w") as f:
            json.dump(res, f, indent=1)
            f.write("\n")
        print(json.dumps(res))
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the quantize / dequantize path "
              "runs on a single device with no collectives; --gpus must be 1.",
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch

    from communication_efficient_gradient_amd import gq
    from communication_efficient_gradient_amd import workloads as WL

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    hl = Headline(torch, gq, WL, stream)
    if args.counters:
        for t in range(2):
            hl.step(t)
        # calibration: one plain elementwise pass (read COPY_BYTES, write
        # COPY_BYTES); torch's negation kernel is the only one of its kind here
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        if args.only:
            hl.release()
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            suite(torch, gq, WL, stream, 1, args.only)
            torch.cuda.synchronize()
            DEFERRED.clear()  # no oracle timings in a counter run
        log("counters run done")
        return 0

    # ---- the timed region: K whole steps, an event around every launch ----
    for t in range(args.warmup):
        hl.step(t)
    torch.cuda.synchronize()
    W = hl.W
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(W + 2)]
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k, t in enumerate(range(args.warmup, args.warmup + args.steps)):
        hl.step(t, evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    gpu_ms_step = evs[0][0].elapsed_time(evs[-1][-1]) / args.steps
    q_durs = [ev[w].elapsed_time(ev[w + 1]) for ev in evs for w in range(W)]
    d_durs = [ev[W].elapsed_time(ev[W + 1]) for ev in evs]
    qs, ds = _stats(q_durs), _stats(d_durs)
    n = hl.n
    qb, db = hl.qbytes(), hl.dbytes()
    achieved = qb / (qs["mean"] * 1e-3) / 1e9
    traffic = load_traffic(Headline.KEY, "k_stream_quant")
    agg_traffic = load_traffic(Headline.AGG_KEY, "k_deq_acc")
    log(f"headline: {ms_step * 1e3:.1f} us/step wall ({gpu_ms_step * 1e3:.1f} us "
        f"GPU); quantize mean {qs['mean'] * 1e3:.1f} us median "
        f"{qs['median'] * 1e3:.1f} us ({achieved:.0f} GB/s); aggregate mean "
        f"{ds['mean'] * 1e3:.1f} us")

    def live(name, st, nbytes, elements):
        r = entry(name, st["median"], nbytes, elements)
        r.update({"ms_mean": round(st["mean"], 5), "ms_p10": round(st["p10"], 5),
                  "ms_p90": round(st["p90"], 5), "runs": st["runs"],
                  "timed": "inside the headline's timed region"})
        return r

    kernels = [
        live(f"quantize int8+ef d=512 n={n} (headline, per worker)", qs, qb, n),
        live(f"dequantize_accumulate int8 W={W} n={n} (headline)", ds, db, n * W),
    ]
    kernels[0].update(oracle_rate(hl.host[0], dict(scheme=0, d=512, s=127),
                                  True, seed=1))
    job = kernels[0].pop("_oracle")
    DEFERRED.append((kernels[0], job))
    kernels[1]["traffic"] = agg_traffic
    if args.suite == "all":
        hl.release()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        kernels.append(copy_reference(torch, stream))
        torch.cuda.empty_cache()
        kernels += suite(torch, gq, WL, stream, args.reps, args.only)
    # every HBM-bound entry also as a fraction of the plain copy of this run
    ref = next((k for k in kernels if k["kernel"].startswith("reference copy")), None)
    if ref is not None:
        for k in kernels:
            if k.get("bound") == "hbm" and k is not ref:
                k["copy_frac"] = round(k["moved_GBps"] / ref["moved_GBps"], 4)
    # host work after every GPU timing (see DEFERRED)
    torch.cuda.synchronize()
    run_deferred()
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(hl)
        log(f"cpu baseline: {cpu}")

    inputs = check_inputs(WL, {
        f"worker {w}": (hl.host[w - 1], lambda r, w=w: r["workers"][w - 1])
        for w in range(1, hl.W + 1)})

    line = {
        "metric": METRIC,
        "value": round(4 * n * W / (ms_step * 1e-3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{W} simulated workers x {n} fp32 elements "
                         "(N(0,1e-3^2) own + shared component): INT8 (s=127) "
                         "+ error feedback, d=512, Philox rounding, then the "
                         f"W={W} dequantize-accumulate average; one step = "
                         f"{W} quantizes + 1 aggregation"),
            "elements_per_worker": n, "workers": W, "bucket": 512,
            "code_bits": hl.bits,
            "hbm_bytes_per_step": W * qb + db,
            "gpu_ms_per_step": round(gpu_ms_step, 5),
            "hbm_frac_per_step": round((W * qb + db) / (ms_step * 1e-3) / 1e9
                                       / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_stream_quant (INT8 s=127, error feedback, d=512)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": qb,
            "avg_launch_us": round(qs["mean"] * 1e3, 3),
            "median_launch_us": round(qs["median"] * 1e3, 3),
            "p10_p90_launch_us": [round(qs["p10"] * 1e3, 3),
                                  round(qs["p90"] * 1e3, 3)],
            "launches": qs["runs"],
        },
        "cpu_baseline": cpu,
        "parity_full_size": load_parity(),
        "cpu_oracle_full_size": load_cpu_configs(),
        "inputs": inputs,
        "kernels": kernels,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
