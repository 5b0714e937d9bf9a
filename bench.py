"""Benchmark of the deterministic W8A8 hot path on one MI355X.

One step is one pass of the whole path over a long-evidence prefill batch
(M = 8192 tokens, hidden 5120, intermediate 17408, an lm_head of 248000
rows):

  quantize x [8192,5120]  -> gate+up GEMM  5120 -> 34816
  quantize h [8192,17408] -> down GEMM    17408 -> 5120, + residual, split-K S
  quantize the answer row -> candidate read-out, C = 4 lm_head rows

The inputs are seeded synthetic data with the decision model's shapes.  They
are resident in HBM before the timed region starts.  ``value`` is the int8
tera-operations (2*M*N*K per GEMM) per second of the whole step.
``roofline`` is for the dominant kernel (the gate+up GEMM) against the int8
MFMA peak.  Its duration is measured with HIP events around every launch of
that kernel inside the timed steps.  ``readout`` reports the full-vocabulary
skinny GEMM (M = 3 answer rows x 248000 lm_head rows), which is HBM-bound,
against HBM bandwidth.  That is the general path the candidate read-out
replaces, timed in the same run; ``readout.candidates_us`` is the
candidate-only read-out of the same rows (C candidates each), with events
around each launch (for so short a kernel that is mostly the host's time
per call) and back to back, and ``candidates_speedup_vs_full`` the full
read-out's time over the back-to-back one.  ``mfma_ceiling`` is the throughput the
int8 matrix cores sustain on register-resident operands with no memory
traffic (uniform int8, and activation-like A; 32x32x32 and 16x16x64 MFMAs),
measured in the same run; ``roofline.frac_of_sustained_ceiling`` relates
the GEMM to the ceiling of its own MFMA form on activation-like operands.
``cpu_baseline`` is the CPU oracle on a bounded sample of the same step
(rank 0 only): the first R tokens through both layers and the read-out of
token R-1, on all host threads and single-threaded, with the CPU model.
``parity`` compares the GPU's outputs of those rows with the oracle's, bit
for bit (the answer head is run once more on row R-1 for it).
``large_m_config4`` times the batch-invariance stress batch (64 requests,
M = 17664 with padding) through 5120 -> 15360 at split-K 1 and 4.
``mid_m`` reports each mid-sized projection both with events around every
launch and as 30 launches back to back.  ``readout.answer_head_us`` is the
answer head's device time per launch: 50 launches queued behind three
GEMMs, two events around the 50 (what a kernel trace reports for it);
``answer_head_us_events_each`` is the same kernel with events around each
launch of the step (adds the events' own cost), and
``answer_head_host_us_per_call`` the host time the binding takes per call.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--splitk S]
                       [--legs all|none|splitk,readout,...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
METRIC = "W8A8 GEMM TOPS and % int8 MFMA peak (bit-exact); read-out GB/s % HBM"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "gemm_tiled": os.path.join(ROOT, "deterministic_w8a8_int8_amd", "csrc", "gemm_tiled.hip"),
    "gemm_skinny": os.path.join(ROOT, "deterministic_w8a8_int8_amd", "csrc", "gemm_skinny.hip"),
    "quantize": os.path.join(ROOT, "deterministic_w8a8_int8_amd", "csrc", "quantize.hip"),
}


def source_sha(name: str) -> str:
    with open(KERNEL_SOURCES[name], "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(key: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; None otherwise."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[key]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_sha") != source_sha(kernel):
        return None
    return t["bytes_per_launch"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--splitk", type=int, default=1, help="split-K factor of the down projection")
    ap.add_argument("--M", type=int, default=8192, help="prefill tokens")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--legs", default="all",
                    help="comma list of the legs run after the timed steps: splitk, readout, stream, mid_m, "
                         "config4, row_parallel, graph, requant, ceiling, cpu; 'all' (default) or 'none' "
                         "(shorter runs under a profiler)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


class Timer:
    """HIP events around kernel launches on the current stream, per name."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, name, fn):
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        out = fn()
        e1.record()
        self.pairs.setdefault(name, []).append((e0, e1))
        return out

    def mean_us(self, name):
        ps = self.pairs.get(name, [])
        return 1e3 * float(np.mean([a.elapsed_time(b) for a, b in ps])) if ps else None

    def pct_us(self, name):
        """Median, 10th and 90th percentile of the launch durations (us)."""
        ts = np.array([1e3 * a.elapsed_time(b) for a, b in self.pairs.get(name, [])])
        if ts.size == 0:
            return None
        p10, p50, p90 = np.percentile(ts, [10, 50, 90])
        return {"median": round(float(p50), 2), "p10": round(float(p10), 2), "p90": round(float(p90), 2)}

    def clear(self):
        self.pairs = {}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(gu, dn, head, cand, seconds):
    """The CPU oracle, untuned, on the first R rows of both layers plus the
    answer read-out of row R-1; R grows until the sample costs about
    `seconds` on all threads.  Also the same work single-threaded on a
    smaller sample.  Returns (baseline, outputs): the oracle's outputs of the
    sample are what the GPU's rows are checked against."""
    import oracle

    def work(R):
        t0 = time.perf_counter()
        xq, sx = oracle.quantize_act(gu["x"][:R], gu["smooth"])
        y1 = oracle.gemm(xq, sx, gu["w"], gu["sw"])
        xq2, sx2 = oracle.quantize_act(dn["x"][:R], dn["smooth"])
        y2 = oracle.gemm(xq2, sx2, dn["w"], dn["sw"], dn["r"][:R])
        xq3, sx3 = oracle.quantize_act(y2[-1:], head["smooth"])
        logits, _ = oracle.readout_candidates(xq3, sx3, head["w"], head["sw"], cand)
        probs = oracle.candidate_softmax(logits)
        dt = time.perf_counter() - t0
        return dt, {"R": R, "xq1": xq, "sx1": sx, "y1": y1, "xq2": xq2, "sx2": sx2, "y2": y2,
                    "logits": logits, "probs": probs}

    K1, N1, K2, N2 = gu["K"], gu["N"], dn["K"], dn["N"]
    ops = lambda R: 2.0 * R * (N1 * K1 + N2 * K2) + 2.0 * cand.size * head["K"]
    threads = oracle.num_threads()
    R = threads
    dt, _ = work(R)
    R = int(min(gu["M"], max(threads, threads * round(seconds / max(dt, 1e-3)))))
    dt, out = work(R)
    # single thread, on a sample about 1/threads as large
    R1 = max(1, R // max(threads, 1))
    oracle.set_num_threads(1)
    try:
        dt1, _ = work(R1)
    finally:
        oracle.set_num_threads(threads)
    base = {"value": round(ops(R) / dt / 1e12, 6), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(),
            "single_thread_TOPS": round(ops(R1) / dt1 / 1e12, 6),
            "sample": f"first {R} of {gu['M']} tokens through both layers plus the read-out of row {R - 1} "
                      f"({ops(R) / 1e9:.1f} GOP in {dt:.2f} s on {threads} threads, int64 scalar loops); "
                      f"single thread: first {R1} tokens ({ops(R1) / 1e9:.1f} GOP in {dt1:.2f} s)"}
    return base, out


def parity_against_oracle(torch, B, out, xq1, sx1, y1, xq2, sx2, y2, wh, swh, sh, cand_d):
    """The GPU's outputs of the rows the CPU baseline computed, bit for bit:
    quantised activations and scales of both layers, both layers' outputs,
    and the answer head run on row R-1 of the GPU's down-projection output
    (candidate logits bit for bit, probabilities within 2^-44)."""
    R = out["R"]
    checks = {}

    def cmp_bits(name, got, want):
        got, want = np.ascontiguousarray(got), np.ascontiguousarray(want)
        if got.shape != want.shape or got.itemsize != want.itemsize:
            checks[name] = (int(want.size), int(want.size))
            return
        u = {1: np.uint8, 4: np.uint32, 8: np.uint64}[want.itemsize]
        checks[name] = (int(want.size), int((got.view(u) != want.view(u)).sum()))

    cmp_bits("xq1", xq1[:R].cpu().numpy(), out["xq1"])
    cmp_bits("sx1", sx1[:R].cpu().numpy(), out["sx1"])
    cmp_bits("y1", y1[:R].cpu().numpy(), out["y1"])
    cmp_bits("xq2", xq2[:R].cpu().numpy(), out["xq2"])
    cmp_bits("sx2", sx2[:R].cpu().numpy(), out["sx2"])
    cmp_bits("y2", y2[:R].cpu().numpy(), out["y2"])
    rows = torch.tensor([R - 1], dtype=torch.int32, device="cuda")
    logits, probs = B.w8a8_answer_head(y2, rows, sh, wh, swh, cand_d)
    cmp_bits("logits", logits.cpu().numpy(), out["logits"])
    p = probs.cpu().numpy()
    bad_p = int((np.abs(p - out["probs"]) > 2.0 ** -44 * np.abs(out["probs"])).sum())
    checks["probs_within_2^-44"] = (int(p.size), bad_p)
    return {"checked": sum(c for c, _ in checks.values()), "mismatches": sum(b for _, b in checks.values()),
            "rows": R, "by_output": {k: {"checked": c, "mismatches": b} for k, (c, b) in checks.items()}}


def startup_requantize(torch, B, w1, s1, w2, s2):
    """One-off startup requantisation of Q8_0 weights with SmoothQuant (the
    layer weights stand in for Q8_0 codes, with random binary16 block
    scales): time and GB/s for the gate+up and down weights."""
    out = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    for name, q, s in (("gate_up", w1, s1), ("down", w2, s2)):
        N, K = q.shape
        d = (torch.rand((N, K // 32), device="cuda", generator=g) * 1e-2 + 1e-4).to(torch.float16)
        w = torch.empty_like(q)
        sw = torch.empty((N,), dtype=torch.float32, device="cuda")
        fn = lambda: B.w8a8_requantize_q8_0(q, d, s, w=w, sw=sw)
        for _ in range(2):
            fn()
        t = Timer(torch)
        for _ in range(5):
            t.run("r", fn)
        torch.cuda.synchronize()
        us = t.mean_us("r")
        nbytes = 2 * N * K + 2 * N * (K // 32) + 4 * K + 4 * N
        out[name] = {"shape": [N, K], "us": round(us, 1), "GBs": round(nbytes / (us * 1e-6) / 1e9, 1)}
        del d, w, sw
    return out


def short_request_graph(torch, B, synth):
    """A 256-token request (gate+up, down at split-K 4, answer head over a
    50000-row lm_head: 6 launches, the answer head one of them) run eagerly
    and replayed from one captured HIP graph;
    the answer-head tables stay in device memory, so one capture serves
    every request of the bucket."""
    gu, dn, head = synth.short_request("gate_up"), synth.short_request("down"), synth.lm_head(V=50000)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    M = 256
    x1, s1, w1, sw1 = d(gu["x"]), d(gu["smooth"]), d(gu["w"]), d(gu["sw"])
    x2, s2, w2, sw2, r2 = d(dn["x"]), d(dn["smooth"]), d(dn["w"]), d(dn["sw"]), d(dn["r"])
    wh, swh, sh = d(head["w"]), d(head["sw"]), d(head["smooth"])
    xq1, sx1, y1 = e((M, gu["K"]), torch.int8), e((M,), torch.float32), e((M, gu["N"]), torch.float32)
    xq2, sx2, y2 = e((M, dn["K"]), torch.int8), e((M,), torch.float32), e((M, dn["N"]), torch.float32)
    ws = B.splitk_workspace(M, dn["N"], dn["K"], 4)
    rows = torch.tensor([M - 1], dtype=torch.int32, device="cuda")
    cand = torch.tensor([[3, 17, 4000, 49999]], dtype=torch.int32, device="cuda")
    xq3, sx3 = e((1, dn["N"]), torch.int8), e((1,), torch.float32)
    logits, probs = e((1, 4), torch.float32), e((1, 4), torch.float64)

    def head_only():
        B.w8a8_answer_head(y2, rows, sh, wh, swh, cand, xq=xq3, sx=sx3, logits=logits, probs=probs)

    def step():
        B.w8a8_quantize_act(x1, s1, xq=xq1, sx=sx1)
        B.w8a8_gemm(xq1, sx1, w1, sw1, y=y1)
        B.w8a8_quantize_act(x2, s2, xq=xq2, sx=sx2)
        B.w8a8_gemm_splitk(xq2, sx2, w2, sw2, 4, residual=r2, y=y2, workspace=ws)
        head_only()

    def timed(fn, n=50):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / n

    def isolated(fn, n=50):
        # host wall clock of one call issued on an idle GPU, synchronised
        ts = []
        for _ in range(n):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
        return 1e6 * float(np.median(ts))

    out = {}
    for name, fn in (("step", step), ("answer_head", head_only)):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                fn()
        torch.cuda.current_stream().wait_stream(s)
        eager = timed(fn)
        replay = timed(g.replay)
        out[name] = {"eager_us": round(eager, 1), "graph_us": round(replay, 1),
                     "eager_isolated_us": round(isolated(fn), 1),
                     "graph_isolated_us": round(isolated(g.replay), 1),
                     "launches": 6 if name == "step" else 1}
    return out


def row_parallel_rank(torch, B, x2, s2, w2, sw2, r2):
    """One rank's kernels of the row-parallel down projection (8192 x 5120 x
    17408 split over `ranks`), each timed alone: the slice maximum, the
    quantisation with the global maximum, the int32 partial GEMM of the
    slice, and the epilogue that adds all ranks' partials (what follows the
    int32 all-reduce)."""
    M, K = x2.shape
    N = w2.shape[0]
    out = {}
    for ranks in (2, 8):
        ks = K // ranks
        xs, ss = x2[:, :ks], s2[:ks]
        ws = w2[:, :ks].contiguous()
        amax = B.w8a8_row_absmax(xs, ss)
        xq, sx = B.w8a8_quantize_act_amax(xs, ss, amax)
        parts = torch.empty((ranks, M, N), dtype=torch.int32, device="cuda")
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        fns = {"row_absmax": lambda: B.w8a8_row_absmax(xs, ss, amax=amax),
               "quantize_act_amax": lambda: B.w8a8_quantize_act_amax(xs, ss, amax, xq=xq, sx=sx),
               "gemm_int32": lambda: B.w8a8_gemm_int32(xq, ws, acc=parts[0]),
               "epilogue_int32": lambda: B.w8a8_epilogue_int32(parts, sx, sw2, residual=r2, y=y)}
        res = {}
        for name, fn in fns.items():
            for _ in range(2):
                fn()
            t = Timer(torch)
            for _ in range(10):
                t.run(name, fn)
            torch.cuda.synchronize()
            res[name] = {"us": round(t.mean_us(name), 1)}
        res["row_absmax"]["GBs"] = round(4 * M * ks / (res["row_absmax"]["us"] * 1e-6) / 1e9, 1)
        res["quantize_act_amax"]["GBs"] = round(5 * M * ks / (res["quantize_act_amax"]["us"] * 1e-6) / 1e9, 1)
        res["gemm_int32"]["TOPS"] = round(2.0 * M * N * ks / (res["gemm_int32"]["us"] * 1e-6) / 1e12, 1)
        res["epilogue_int32"]["GBs"] = round((4 * ranks + 8) * M * N / (res["epilogue_int32"]["us"] * 1e-6) / 1e9, 1)
        out[f"{ranks}_ranks"] = {"slice_K": ks, **res}
        del parts, y, ws
    return out


def roof_us_of(M, N, K, res):
    """max(ops / int8 MFMA peak, bytes / HBM peak) in microseconds."""
    ops = 2.0 * M * N * K
    nbytes = M * K + N * K + 4 * (M + N) + 4 * M * N * (2 if res else 1)
    return max(ops / (PEAK_INT8_TOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)) * 1e6


def large_m_config4(torch, B, synth):
    """The batch-invariance stress batch (64 requests of U{32..512} tokens in
    its first arrangement, padded to a multiple of 256) through the
    5120 -> 15360 layer at split-K 1 and 4: time, TOPS and the fraction of the
    int8 MFMA peak.  Inputs are the synthetic requests, quantised on the GPU."""
    reqs, layer = synth.invariance_requests()
    x, _ = synth.arrangement(reqs, 0)
    M, K = x.shape
    N = layer["N"]
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    xq, sx = B.w8a8_quantize_act(d(x), d(layer["smooth"]))
    w, sw = d(layer["w"]), d(layer["sw"])
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    out = {"shape": [int(M), int(N), int(K)], "requests": len(reqs),
           "tokens": int(sum(r.shape[0] for r in reqs))}
    ops = 2.0 * M * N * K
    for S in (1, 4):
        ws = B.splitk_workspace(M, N, K, S) if S > 1 else None
        fn = (lambda: B.w8a8_gemm(xq, sx, w, sw, y=y)) if S == 1 else \
             (lambda: B.w8a8_gemm_splitk(xq, sx, w, sw, S, y=y, workspace=ws))
        for _ in range(3):
            fn()
        t = Timer(torch)
        for _ in range(10):
            t.run("g", fn)
        torch.cuda.synchronize()
        us = t.mean_us("g")
        tops = ops / (us * 1e-6) / 1e12
        out[f"splitk{S}"] = {"us": round(us, 1), "pct_us": t.pct_us("g"), "TOPS": round(tops, 1),
                             "frac_mfma": round(tops / PEAK_INT8_TOPS, 4),
                             "plan": B.w8a8_gemm_plan(M, N, K, S, 0)}
        del ws
    out["roof_us"] = round(roof_us_of(M, N, K, False), 1)
    del xq, sx, w, sw, y
    return out


def mid_m_shapes(torch, B, stream_read_gbs):
    """The short-request (M = 256) and forest-batch (M = 328) projections:
    near the ridge of the int8 roofline, so each reports its time against
    max(ops / MFMA peak, bytes / HBM peak).  Uniform random int8 operands;
    three weight copies are rotated, so the weights stream from HBM rather
    than from the 256 MB last-level cache.  `plan` is the library's kernel
    choice (w8a8_gemm_plan)."""
    shapes = [("short_request_gate_up", 256, 34816, 5120, False, 1),
              ("short_request_down", 256, 5120, 17408, True, 1),
              ("short_request_down_splitk8", 256, 5120, 17408, True, 8),
              ("forest_qkv_like", 328, 15360, 5120, False, 1),
              ("forest_gate_up", 328, 34816, 5120, False, 1)]
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    out = {}
    for name, M, N, K, res, S in shapes:
        xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
        ws3 = [torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g) for _ in range(3)]
        sx = torch.rand(M, device="cuda", generator=g) * 0.01 + 1e-3
        sw = torch.rand(N, device="cuda", generator=g) * 0.01 + 1e-3
        r = torch.randn(M, N, device="cuda", generator=g) if res else None
        y = torch.empty(M, N, device="cuda")
        ws = B.splitk_workspace(M, N, K, S) if S > 1 else None
        it = [0]

        def fn():
            w = ws3[it[0] % 3]
            it[0] += 1
            if S == 1:
                B.w8a8_gemm(xq, sx, w, sw, residual=r, y=y)
            else:
                B.w8a8_gemm_splitk(xq, sx, w, sw, S, residual=r, y=y, workspace=ws)
        for _ in range(3):
            fn()
        t = Timer(torch)
        for _ in range(30):
            t.run("g", fn)
        torch.cuda.synchronize()
        us = t.mean_us("g")
        # the same launches back to back between two events: the time per
        # layer in a stream of layers (no event between launches)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(30):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us_b2b = 1e3 * e0.elapsed_time(e1) / 30
        ops = 2.0 * M * N * K
        nbytes = M * K + N * K + 4 * (M + N) + 4 * M * N * (2 if res else 1)
        roof_us = max(ops / (PEAK_INT8_TOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)) * 1e6
        out[name] = {"shape": [M, N, K], "splitk": S, "plan": B.w8a8_gemm_plan(M, N, K, S, res),
                     "us": round(us, 1), "pct_us": t.pct_us("g"), "us_back_to_back": round(us_b2b, 1),
                     "frac_of_roof_back_to_back": round(roof_us_of(M, N, K, res) / us_b2b, 4),
                     "TOPS": round(ops / (us * 1e-6) / 1e12, 1),
                     "GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "roof_us": round(roof_us, 1), "frac_of_roof": round(roof_us / us, 4),
                     "bound": "hbm" if nbytes / (PEAK_HBM_GBS * 1e9) > ops / (PEAK_INT8_TOPS * 1e12)
                     else "mfma"}
        del xq, ws3, r, y, ws
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by rows or output columns with no communication between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from deterministic_w8a8_int8_amd import binding as B
    from deterministic_w8a8_int8_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    M, S = args.M, args.splitk
    print(f"# generating inputs (M={M})", file=sys.stderr, flush=True)
    gu = synth.long_prefill("gate_up", M=M)
    dn = synth.long_prefill("down", M=M)
    head = synth.lm_head()
    rd = synth.readout_inputs()
    cand1 = rd["cand"][:1]                      # C = 4 candidates for the one answer row
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()

    x1, s1, w1, sw1 = dev(gu["x"]), dev(gu["smooth"]), dev(gu["w"]), dev(gu["sw"])
    x2, s2, w2, sw2, r2 = dev(dn["x"]), dev(dn["smooth"]), dev(dn["w"]), dev(dn["sw"]), dev(dn["r"])
    wh, swh, sh = dev(head["w"]), dev(head["sw"]), dev(head["smooth"])
    cand_d = dev(cand1)
    answer = torch.tensor([M - 1], dtype=torch.int32, device="cuda")
    K1, N1, K2, N2 = gu["K"], gu["N"], dn["K"], dn["N"]
    xq1 = torch.empty((M, K1), dtype=torch.int8, device="cuda")
    sx1 = torch.empty((M,), dtype=torch.float32, device="cuda")
    xq2 = torch.empty((M, K2), dtype=torch.int8, device="cuda")
    sx2 = torch.empty((M,), dtype=torch.float32, device="cuda")
    y1 = torch.empty((M, N1), dtype=torch.float32, device="cuda")
    y2 = torch.empty((M, N2), dtype=torch.float32, device="cuda")
    xq3 = torch.empty((1, K1), dtype=torch.int8, device="cuda")
    sx3 = torch.empty((1,), dtype=torch.float32, device="cuda")
    logits = torch.empty((1, cand1.shape[1]), dtype=torch.float32, device="cuda")
    probs = torch.empty((1, cand1.shape[1]), dtype=torch.float64, device="cuda")
    ws = B.splitk_workspace(M, N2, K2, S) if S > 1 else None
    timer = Timer(torch)

    def step():
        timer.run("quantize_h5120", lambda: B.w8a8_quantize_act(x1, s1, xq=xq1, sx=sx1))
        timer.run("gemm_gate_up", lambda: B.w8a8_gemm(xq1, sx1, w1, sw1, y=y1))
        timer.run("quantize_h17408", lambda: B.w8a8_quantize_act(x2, s2, xq=xq2, sx=sx2))
        if S > 1:
            timer.run("gemm_down", lambda: B.w8a8_gemm_splitk(xq2, sx2, w2, sw2, S, residual=r2, y=y2,
                                                              workspace=ws))
        else:
            timer.run("gemm_down", lambda: B.w8a8_gemm(xq2, sx2, w2, sw2, residual=r2, y=y2))
        timer.run("answer_head",
                  lambda: B.w8a8_answer_head(y2, answer, sh, wh, swh, cand_d, xq=xq3, sx=sx3,
                                             logits=logits, probs=probs))

    print("# warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer.clear()
    print(f"# timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / max(args.steps, 1)
    ops_step = 2.0 * M * (N1 * K1 + N2 * K2) + 2.0 * cand1.size * K1
    value = ops_step / (wall / args.steps) / 1e12
    kernels = {k: round(timer.mean_us(k), 2) for k in timer.pairs}
    kernels_pct = {k: timer.pct_us(k) for k in timer.pairs}
    legs = set(("splitk,readout,stream,mid_m,config4,row_parallel,graph,requant,ceiling,cpu"
                if args.legs == "all" else "" if args.legs == "none" else args.legs).split(","))

    # the answer head back to back: 50 launches queued behind three gate+up
    # GEMMs (about 3.4 ms of device work, longer than the host takes to
    # enqueue the 50), so the device runs them one after another without
    # waiting for the host; the host's own time per call is reported too
    head_fn = lambda: B.w8a8_answer_head(y2, answer, sh, wh, swh, cand_d, xq=xq3, sx=sx3,
                                         logits=logits, probs=probs)
    head_b2b, head_host = [], []
    for _ in range(3):
        for _ in range(3):
            B.w8a8_gemm(xq1, sx1, w1, sw1, y=y1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        h0 = time.perf_counter()
        for _ in range(50):
            head_fn()
        head_host.append(1e6 * (time.perf_counter() - h0) / 50)
        e1.record()
        torch.cuda.synchronize()
        head_b2b.append(1e3 * e0.elapsed_time(e1) / 50)

    # dominant kernel roofline: gate+up GEMM on the int8 MFMA peak
    gu_us = timer.mean_us("gemm_gate_up")
    gu_tops = 2.0 * M * N1 * K1 / (gu_us * 1e-6) / 1e12
    roofline = {"bound": "mfma", "achieved": round(gu_tops, 1), "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                "frac": round(gu_tops / PEAK_INT8_TOPS, 4),
                "traffic": measured_traffic("gemm_gate_up_long_prefill", "gemm_tiled"),
                "kernel": "gemm_tiled ({}x{} tile)".format(*B.w8a8_gemm_plan(M, N1, K1, 1, 0)[2:4]),
                "shape": [M, N1, K1]}
    dn_us = timer.mean_us("gemm_down")
    down = {"us": round(dn_us, 1), "tops": round(2.0 * M * N2 * K2 / (dn_us * 1e-6) / 1e12, 1),
            "splitk": S}
    down["frac_mfma"] = round(down["tops"] / PEAK_INT8_TOPS, 4)
    quant = {}
    for key, K in (("quantize_h5120", K1), ("quantize_h17408", K2)):
        us = timer.mean_us(key)
        gbs = (M * K * 5 + 4 * K + 4 * M) / (us * 1e-6) / 1e9
        quant[key] = {"us": round(us, 1), "GBs": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}

    # down projection at other split-K factors (bit-identical output; timed only)
    split_us = {}
    for s_ in ((1, 2, 4, 8) if "splitk" in legs else ()):
        w_ = B.splitk_workspace(M, N2, K2, s_) if s_ > 1 else None
        fn = (lambda: B.w8a8_gemm(xq2, sx2, w2, sw2, residual=r2, y=y2)) if s_ == 1 else \
             (lambda: B.w8a8_gemm_splitk(xq2, sx2, w2, sw2, s_, residual=r2, y=y2, workspace=w_))
        for _ in range(3):
            fn()
        t = Timer(torch)
        for _ in range(10):
            t.run("d", fn)
        torch.cuda.synchronize()
        split_us[str(s_)] = round(t.mean_us("d"), 1)
        del w_

    readout = {"answer_head_us": round(float(np.median(head_b2b)), 2),
               "answer_head_us_events_each": kernels.get("answer_head"),
               "answer_head_host_us_per_call": round(float(np.median(head_host)), 2)}
    if "readout" in legs:
        print("# leg readout", file=sys.stderr, flush=True)
        # full-vocabulary read-out (M = 3 answer rows): HBM-bound skinny GEMM
        Mr = rd["answer_rows"].size
        xqr, sxr = B.w8a8_quantize_act(dev(rd["h"]), sh, row_idx=dev(rd["answer_rows"]))
        yfull = torch.empty((Mr, head["N"]), dtype=torch.float32, device="cuda")
        for _ in range(3):
            B.w8a8_gemm(xqr, sxr, wh, swh, y=yfull)
        t = Timer(torch)
        for _ in range(20):
            t.run("full", lambda: B.w8a8_gemm(xqr, sxr, wh, swh, y=yfull))
        torch.cuda.synchronize()
        full_us = t.mean_us("full")
        full_bytes = head["N"] * head["K"] + 4 * head["N"] + Mr * head["K"] + 4 * Mr + 4 * Mr * head["N"]
        full_gbs = full_bytes / (full_us * 1e-6) / 1e9
        # the same rows' candidate-only read-out (C candidates each)
        cand3 = dev(rd["cand"])
        lg3 = torch.empty(tuple(rd["cand"].shape), dtype=torch.float32, device="cuda")
        for _ in range(3):
            B.w8a8_readout_candidates(xqr, sxr, wh, swh, cand3, logits=lg3)
        for _ in range(20):
            t.run("cand", lambda: B.w8a8_readout_candidates(xqr, sxr, wh, swh, cand3, logits=lg3))
        torch.cuda.synchronize()
        cand_us = t.mean_us("cand")
        # back to back: 50 launches queued behind six full read-outs (about
        # 1.1 ms of device work, longer than the host takes to enqueue them)
        cand_b2b = []
        for _ in range(3):
            for _ in range(6):
                B.w8a8_gemm(xqr, sxr, wh, swh, y=yfull)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(50):
                B.w8a8_readout_candidates(xqr, sxr, wh, swh, cand3, logits=lg3)
            e1.record()
            torch.cuda.synchronize()
            cand_b2b.append(1e3 * e0.elapsed_time(e1) / 50)
        cand_b2b_us = float(np.median(cand_b2b))
        readout = {"bound": "hbm", "achieved": round(full_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": round(full_gbs / PEAK_HBM_GBS, 4), "us": round(full_us, 1),
                   "shape": [int(Mr), head["N"], head["K"]], "kernel": "gemm_skinny",
                   "traffic": measured_traffic("gemm_full_vocab_readout", "gemm_skinny"),
                   "candidates_us": round(cand_us, 2), "candidates_us_back_to_back": round(cand_b2b_us, 2),
                   "candidates_shape": [int(x) for x in rd["cand"].shape],
                   "candidates_speedup_vs_full": round(full_us / cand_b2b_us, 1), **readout}
        del yfull, lg3

    best_read = None
    if "stream" in legs:
        print("# leg stream", file=sys.stderr, flush=True)
        # streaming read of 4 GiB: the read bandwidth HBM sustains on this GPU
        rbuf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
        rsink = torch.zeros(4, dtype=torch.int32, device="cuda")
        B.w8a8_probe_stream_read(rbuf, rsink)
        best_read = 0.0
        for _ in range(5):
            t = Timer(torch)
            nbytes = t.run("r", lambda: B.w8a8_probe_stream_read(rbuf, rsink))
            torch.cuda.synchronize()
            best_read = max(best_read, nbytes / (t.mean_us("r") * 1e-6) / 1e9)
        del rbuf
        readout["stream_read_GBs"] = round(best_read, 1)
        if "achieved" in readout:
            readout["frac_of_stream_read"] = round(readout["achieved"] / best_read, 4)
        for q in quant.values():
            q["frac_of_stream_read"] = round(q["GBs"] / best_read, 4)
        # the quantizer's traffic mix alone (4 bytes read, 1 written per
        # element) at its two sizes, sources rotated over three copies so the
        # reads come from HBM: the rate any quantizer moving these bytes meets
        for key, K in (("quantize_h5120", K1), ("quantize_h17408", K2)):
            srcs = [torch.empty(M * K, dtype=torch.float32, device="cuda").normal_() for _ in range(3)]
            dst = torch.empty(M * K, dtype=torch.int8, device="cuda")
            for i in range(3):
                B.w8a8_probe_stream_narrow(srcs[i], dst)
            t = Timer(torch)
            for i in range(30):
                moved = t.run("n", lambda: B.w8a8_probe_stream_narrow(srcs[i % 3], dst))
            torch.cuda.synchronize()
            narrow_gbs = moved / (t.mean_us("n") * 1e-6) / 1e9
            quant[key]["stream_narrow_GBs"] = round(narrow_gbs, 1)
            quant[key]["frac_of_stream_narrow"] = round(quant[key]["GBs"] / narrow_gbs, 4)
            del srcs, dst

    def leg(name, fn):
        if name not in legs:
            return None
        print(f"# leg {name}", file=sys.stderr, flush=True)
        return fn()

    mid_m = leg("mid_m", lambda: mid_m_shapes(torch, B, best_read))
    config4 = leg("config4", lambda: large_m_config4(torch, B, synth))
    row_parallel = leg("row_parallel", lambda: row_parallel_rank(torch, B, x2, s2, w2, sw2, r2))
    graph = leg("graph", lambda: short_request_graph(torch, B, synth))
    requant = leg("requant", lambda: startup_requantize(torch, B, w1, s1, w2, s2))

    # sustained MFMA-only ceiling on this GPU for two kinds of operand data and
    # both MFMA forms; the large-M kernel runs 16x16x64
    ceiling = {}
    if "ceiling" in legs:
        print("# leg ceiling", file=sys.stderr, flush=True)
        sink = torch.zeros(16, dtype=torch.int32, device="cuda")
        for kind, name in ((0, "uniform_int8"), (1, "activation_like"), (2, "uniform_int8_16x16x64"),
                           (3, "activation_like_16x16x64")):
            B.w8a8_probe_mfma_ceiling(kind, 1024, 50, sink)
            best = 0.0
            for _ in range(3):
                t = Timer(torch)
                ops = t.run("c", lambda: B.w8a8_probe_mfma_ceiling(kind, 1024, 1500, sink))
                torch.cuda.synchronize()
                best = max(best, ops / (t.mean_us("c") * 1e-6) / 1e12)
            ceiling[name + "_TOPS"] = round(best, 1)
        roofline["sustained_mfma_ceiling_TOPS"] = ceiling["activation_like_16x16x64_TOPS"]
        roofline["frac_of_sustained_ceiling"] = round(gu_tops / ceiling["activation_like_16x16x64_TOPS"], 4)

    cpu, parity = None, None
    if not args.no_cpu_baseline and "cpu" in legs:
        print("# cpu baseline (oracle) and parity of the same rows", file=sys.stderr, flush=True)
        cpu, out = cpu_baseline(gu, dn, head, cand1, args.cpu_seconds)
        parity = parity_against_oracle(torch, B, out, xq1, sx1, y1, xq2, sx2, y2, wh, swh, sh, cand_d)
        del out

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8 (int32 accumulate, fp32 epilogue)",
        "data": "synthetic",
        "config": {"workload": "long-evidence prefill", "M": M, "hidden": K1, "gate_up": N1,
                   "intermediate": K2, "down": N2, "splitk_down": S, "lm_head_rows": head["N"],
                   "candidates": int(cand1.shape[1]), "answer_rows": 1},
        "roofline": roofline, "cpu_baseline": cpu, "parity": parity, "readout": readout, "down": down,
        "quantize": quant, "down_splitk_us": split_us, "kernels_us": kernels,
        "kernels_us_pct": kernels_pct, "mfma_ceiling": ceiling, "mid_m": mid_m,
        "large_m_config4": config4,
        "row_parallel_rank": row_parallel, "short_request_graph": graph,
        "startup_requantize_q8_0": requant,
    }
    print(json.dumps(line), flush=True)

    if args.copy_probe_mb:
        n = args.copy_probe_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copy probe: {n} bytes read and {n} bytes written per copy, 3 copies",
              file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
