#!/usr/bin/env python3
"""Benchmark of the low-bit-weight matmul hot path on one MI355X.

One JSON line on stdout. Headline (``value``): the W4A16 decode GEMV at M=1,
N=K=4096 (group-128 uINT4 weights, fp16 activations, fp16 output) in GB/s of
algorithmic bytes, timed over exactly ``--steps`` calls replayed from one
captured HIP graph. The line's ``roofline`` carries the same GEMV at the two
11008-sized projection shapes and, for each of the three, a plain streaming
read of the same weight bytes through the same protocol (the achievable
rate). The W4A8 prefill GEMM (M=2048, N=11008, K=4096) is reported in TOPS
under ``prefill``.

Cold weights: every call reads its weights from one of R copies (>= 1 GiB in
rotation), and 1 GiB of other memory is read and written between the untimed
replay and the timed one, so that no call of the timed region finds its
weights in the 256 MB last-level cache, whatever the step count. Steady
state: right before the timed replay, a graph of the same calls over a
separate set of weight copies runs for about WARM_US microseconds, so that
the timed steps start on a busy, clocked-up GPU and the graph's launch is
queued behind it.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-prefill]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4 GEMV HBM GB/s (% peak) at M=1; W4A8 GEMM TOPS (% MFMA peak) at M=2048"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
I8_PEAK_TOPS = 5000.0          # MI355X dense INT8 MFMA
LLC_BYTES = 256 << 20          # MI355X last-level (Infinity) cache
ROTATE_BYTES = 1 << 30         # weight copies in rotation per workload
FLUSH_BYTES = 1 << 30          # read between the untimed and the timed pass
PREFILL_MIN_STEPS = 50         # the prefill is timed over at least this many calls
CALIB_BYTES = 256 << 20        # device-to-device copy used to calibrate PMC byte counters
PROBE_PER = (1, 2, 4, 8)       # 16-byte loads per lane tried by the read probe
WARM_US = 250.0                # GPU time of the warm-up replay right before a timed one
WARM_COPIES = 8                # weight copies the warm-up replay cycles through
PROFILES = os.path.join(ROOT, "profiles")
def decode_traffic_path(N, K):
    """The committed PMC traffic summary of the W4A16 M=1 GEMV at (N, K)."""
    return os.path.join(PROFILES, f"k_gemv_w4a16_decode_m1_n{N}_k{K}_traffic.json")


DECODE_TRAFFIC = decode_traffic_path(4096, 4096)
PREFILL_TRAFFIC = os.path.join(PROFILES, "k_gemm_w4a8_prefill_m2048_n11008_k4096_traffic.json")
DECODE_SHAPES = ((4096, 4096), (11008, 4096), (4096, 11008))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(M, N, K):
    """Algorithmic bytes of one W4A16 call: packed W + fp16 scales + uint8
    zeros + fp16 A + fp16 C."""
    G = K // 128
    return N * K // 2 + N * G * 2 + N * G + M * K * 2 + M * N * 2


def prefill_bytes(M, N, K):
    """Algorithmic bytes of one W4A8 GEMM call: packed W + fp32 w_scale +
    int8 A + fp32 a_scale + fp16 bias + fp16 C."""
    return N * K // 2 + N * 4 + M * K + M * 4 + N * 2 + M * N * 2


def rotation(copy_bytes):
    """Number of weight copies whose total reaches ROTATE_BYTES."""
    return max(1, math.ceil(ROTATE_BYTES / copy_bytes))


def cold_gap_bytes(steps, copies, copy_bytes, flush_bytes=FLUSH_BYTES):
    """Fewest bytes that pass through memory between two reads of one weight
    copy inside a timed region of `steps` calls over `copies` copies: the
    flush before the region for each copy's first read there, the other
    copies for a read that comes round again. Above the last-level cache
    size, every timed call reads its weights from HBM."""
    gap = flush_bytes
    if steps > copies:
        gap = min(gap, (copies - 1) * copy_bytes)
    return gap


class Flush:
    """Reads FLUSH_BYTES of a buffer of its own with the library's streaming
    read (w4_read_probe, which stores nothing but a conditional sink word),
    evicting the weights from the last-level cache. A read-only flush leaves
    the cache holding clean lines: a flush that wrote would leave dirty ones,
    whose write-back the next reads would pay for (the timed calls would then
    move twice their bytes until the dirty data had drained)."""

    def __init__(self, dev):
        import torch
        self.buf = torch.ones(FLUSH_BYTES, dtype=torch.int8, device=dev)
        self.sink = torch.zeros(1024, dtype=torch.int32, device=dev)

    def __call__(self, stream):
        import torch
        import gemv_nibble_unpack_amd as G
        with torch.cuda.stream(stream):
            G.w4_read_probe(self.buf, FLUSH_BYTES, 8, self.sink)


def warm_steps(step_ms):
    """Steps of a warm-up replay that lasts about WARM_US."""
    return max(2, min(400, math.ceil(WARM_US * 1e-3 / max(step_ms, 1e-6))))


def time_graph(fn, steps, warmup, stream, flush, warm_fn=None):
    """Capture `steps` calls fn(0..steps-1) in one HIP graph and replay it
    once untimed; then flush the last-level cache, replay a warm-up graph of
    warm_fn calls (over other weight copies, about WARM_US long), and time one
    replay of the first graph with HIP events on `stream`; returns ms per
    call. The calls take the current stream (the capture stream while
    capturing)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    gw = None
    if warm_fn is not None:
        nw = warm_steps(t0.elapsed_time(t1) / steps)
        gw = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw):
            for i in range(nw):
                warm_fn(i)
        gw.replay()
    flush(stream)
    if gw is not None:
        gw.replay()
    t0.record(stream)
    g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_eager(fn, steps, warmup, stream, flush):
    """The same calls launched one by one from Python (host launch cost
    included); returns ms per call."""
    import torch
    for i in range(warmup):
        fn(i)
    flush(stream)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        fn(warmup + i)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def calibration_copy():
    """A plain copy kernel of CALIB_BYTES (read once, written once), three
    times: torch's elementwise bitwise_not on uint8 (a device kernel, unlike
    copy_, which the runtime may hand to a DMA engine). Its PMC
    FETCH_SIZE/WRITE_SIZE readings calibrate the byte counters."""
    import torch
    src = torch.ones(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()


def copies_of(Wp):
    """The timed rotation of weight copies (>= ROTATE_BYTES in all), and
    WARM_COPIES more for the warm-up replays (never read in a timed region)."""
    R = rotation(Wp.numel())
    return [Wp] + [Wp.clone() for _ in range(R - 1)], [Wp.clone() for _ in range(WARM_COPIES)]


def read_probe(copies, warm, steps, warmup, stream, flush):
    """The plain streaming read of the same weight copies, in the same
    protocol, at each loads-per-lane setting; the fastest is the achievable
    rate for a transfer of that size."""
    import torch
    import gemv_nibble_unpack_amd as G
    sink = torch.zeros(1024, dtype=torch.int32, device=copies[0].device)
    nbytes = copies[0].numel()
    R, Wn = len(copies), len(warm)
    runs = {}
    for per in PROBE_PER:
        ms = time_graph(lambda i: G.w4_read_probe(copies[i % R], nbytes, per, sink), steps,
                        warmup, stream, flush,
                        warm_fn=lambda i: G.w4_read_probe(warm[i % Wn], nbytes, per, sink))
        runs[per] = ms
    per = min(runs, key=runs.get)
    ms = runs[per]
    return {"bytes": nbytes, "loads_per_lane": per, "us": round(ms * 1e3, 3),
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "us_by_loads_per_lane": {str(k): round(v * 1e3, 3) for k, v in runs.items()}}


def bench_decode_shape(N, K, steps, warmup, stream, flush, eager=False, probe=True):
    """W4A16 M=1 GEMV at (N, K): graph-replay time per call (cold weights),
    the eager rate beside it, and the read probe on the same copies."""
    import torch
    import gemv_nibble_unpack_amd as G
    from gemv_nibble_unpack_amd import workloads as WL
    dev = torch.device("cuda:0")
    if (N, K) == (4096, 4096):
        c = WL.W4A16_DECODE
    else:
        c = next(x for x in WL.W4A16_SWEEP if (x.M, x.N, x.K) == (1, N, K))
    d = c.inputs()
    W = torch.from_numpy(d["W"]).to(dev)
    A = torch.from_numpy(d["A"]).to(dev)
    t = time.time()
    Wq, s, z = G.quantize_pack_w4(W, G.W4_ASYM_GROUP)
    Wp = G.prepack_w(G.W4_LAYOUT_W4A16, Wq, c.N, c.K, s, z)
    torch.cuda.synchronize()
    prep_ms = (time.time() - t) * 1e3
    del W, Wq, s, z
    copies, warm = copies_of(Wp)
    R, Wn = len(copies), len(warm)
    C = torch.empty((c.M, c.N), dtype=torch.float16, device=dev)
    ws = G.Workspace(dev)

    def step(i):
        # stream=None: the current stream (the capture stream under graph capture)
        G.w4a16_gemm(A, copies[i % R], c.N, workspace=ws, C=C)

    def warm_step(i):
        G.w4a16_gemm(A, warm[i % Wn], c.N, workspace=ws, C=C)

    eager_ms = time_eager(step, steps, warmup, stream, flush)
    ms = eager_ms if eager else time_graph(step, steps, warmup, stream, flush, warm_step)
    nbytes = decode_bytes(c.M, c.N, c.K)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"N": c.N, "K": c.K, "bytes": nbytes, "us": round(ms * 1e3, 3),
           "GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
           "eager_us": round(eager_ms * 1e3, 3), "copies": R,
           "cold_gap_bytes": cold_gap_bytes(steps, R, Wp.numel()),
           "offline_prep_ms": round(prep_ms, 3), "ms": ms}
    if probe:
        pr = read_probe(copies, warm, steps, warmup, stream, flush)
        out["achievable"] = pr
        out["frac_of_achievable"] = round(gbs / pr["GBps"], 4)
    del copies, warm
    torch.cuda.empty_cache()
    return out


def bench_prefill(args, stream, flush):
    """W4A8 M=2048 N=11008 K=4096 with fp16 output and bias: the GEMM alone,
    quantize_a8 + GEMM (two calls), and w4a8_gemm_fused_act (one call), each
    replayed from a captured graph over at least PREFILL_MIN_STEPS calls."""
    import torch
    import gemv_nibble_unpack_amd as G
    from gemv_nibble_unpack_amd import workloads as WL

    c = WL.W4A8_PREFILL
    d = c.inputs()
    dev = torch.device("cuda:0")
    W = torch.from_numpy(d["W"]).to(dev)
    A = torch.from_numpy(d["A"]).to(dev)
    bias = torch.from_numpy(d["bias"]).to(dev)
    Wq, wsc, _ = G.quantize_pack_w4(W, G.W4_SYM_PER_CHANNEL)
    Wp = G.prepack_w(G.W4_LAYOUT_W4A8, Wq, c.N, c.K)
    del W, Wq
    copies, warm = copies_of(Wp)
    R, Wn = len(copies), len(warm)
    Aq = torch.empty((c.M, c.K), dtype=torch.int8, device=dev)
    sa = torch.empty(c.M, dtype=torch.float32, device=dev)
    C = torch.empty((c.M, c.N), dtype=torch.float16, device=dev)
    wsp = G.Workspace(dev)
    wsf = G.Workspace(dev)
    steps = max(PREFILL_MIN_STEPS, args.steps // 4)
    warm_n = max(2, args.warmup // 4)
    G.quantize_a8(A, with_rowsum=False, out=(Aq, sa, None))

    def gemm(i, cps=copies):
        G.w4a8_gemm(Aq, sa, cps[i % len(cps)], wsc, c.N, bias=bias, out_dtype=G.W4_OUT_F16,
                    workspace=wsp, C=C)

    def two_calls(i, cps=copies):
        G.quantize_a8(A, with_rowsum=False, out=(Aq, sa, None))
        gemm(i, cps)

    def fused(i, cps=copies):
        G.w4a8_gemm_fused_act(A, cps[i % len(cps)], wsc, c.N, bias=bias, out_dtype=G.W4_OUT_F16,
                              workspace=wsf, C=C)

    def quant(i, cps=None):
        G.quantize_a8(A, with_rowsum=False, out=(Aq, sa, None))

    out = {"steps": steps, "copies": R, "bytes": prefill_bytes(c.M, c.N, c.K),
           "cold_gap_bytes": cold_gap_bytes(steps, R, Wp.numel())}
    if args.eager:
        timer = lambda fn: time_eager(fn, steps, warm_n, stream, flush)
    else:
        timer = lambda fn: time_graph(fn, steps, warm_n, stream, flush,
                                      lambda i: fn(i, warm))
        timer(gemm)           # the first pass over a process's fresh copies runs slow: settle
    out["gemm_ms"] = timer(gemm)
    out["two_call_step_ms"] = timer(two_calls)
    out["fused_step_ms"] = timer(fused)
    out["quant_only_ms"] = timer(quant)
    del copies, warm
    torch.cuda.empty_cache()
    return c, out


def bench_decode_w4a8(stream, steps, flush):
    """W4A8 M=1 N=K=4096 (fp16 activations): quantize_a8 + w4a8_gemm against
    w4a8_gemm_fused_act (graph replay, cold weights)."""
    import torch
    import gemv_nibble_unpack_amd as G
    dev = torch.device("cuda:0")
    N = K = 4096
    rng = np.random.default_rng(700)
    W = torch.from_numpy(rng.normal(0, 0.02, (N, K)).astype(np.float32)).to(dev)
    A = torch.from_numpy(rng.normal(0, 1, (1, K)).astype(np.float16)).to(dev)
    Wq, wsc, _ = G.quantize_pack_w4(W, G.W4_SYM_PER_CHANNEL)
    Wp = G.prepack_w(G.W4_LAYOUT_W4A8, Wq, N, K)
    del W, Wq
    copies, warm = copies_of(Wp)
    C = torch.empty((1, N), dtype=torch.float16, device=dev)
    q = (torch.empty((1, K), dtype=torch.int8, device=dev), torch.empty(1, device=dev), None)
    ws = G.Workspace(dev)

    def two(i, cps=copies):
        G.quantize_a8(A, out=q)
        G.w4a8_gemm(q[0], q[1], cps[i % len(cps)], wsc, N, workspace=ws, C=C)

    def fused(i, cps=copies):
        G.w4a8_gemm_fused_act(A, cps[i % len(cps)], wsc, N, workspace=ws, C=C)

    nb = N * K // 2 + 4 * N + 2 * K + 2 * N
    row = {"N": N, "K": K, "bytes": nb}
    for name, fn in (("two_launch", two), ("fused", fused)):
        ms = time_graph(fn, steps, 10, stream, flush, lambda i, fn=fn: fn(i, warm))
        row[name] = {"us": round(ms * 1e3, 3), "GBps": round(nb / (ms * 1e-3) / 1e9, 1)}
    del copies, warm
    torch.cuda.empty_cache()
    return row


def traffic_of(path):
    """HBM bytes per launch from the committed PMC summary, or None when the
    summary is missing or the kernel sources changed since it was taken."""
    from gemv_nibble_unpack_amd.profiling import load_traffic
    rec = load_traffic(path)
    return None if rec is None else round(rec["traffic_bytes_per_launch"])


def bench_case(case, steps, warmup, stream, flush):
    """Time one workload case (cold weights, steps replayed from one captured
    HIP graph); returns a dict for --sweep."""
    import torch
    import gemv_nibble_unpack_amd as G
    dev = torch.device("cuda:0")
    d = case.inputs()
    A = torch.from_numpy(d["A"]).to(dev)
    M, N, K = case.M, case.N, case.K
    ws = G.Workspace(dev)
    if case.scheme == "w2a16":
        Wq = G.quantize_pack_w2(torch.from_numpy(d["codes"]).to(dev))
        Wp = G.prepack_w(G.W4_LAYOUT_W2A8, Wq, N, K)
        wsc = G.ternary_scale_f16(torch.from_numpy(d["src"]).to(dev))
        nbytes = N * K // 4 + 2 + 2 * M * K + 2 * M * N
        C = torch.empty((M, N), dtype=torch.float16, device=dev)
        copies, warm = copies_of(Wp)
        fn = lambda i, cps=copies: G.w2a16_gemm(A, cps[i % len(cps)], wsc, N, workspace=ws, C=C)
    elif case.scheme == "w4a16":
        Wq, s, z = G.quantize_pack_w4(torch.from_numpy(d["W"]).to(dev), G.W4_ASYM_GROUP)
        Wp = G.prepack_w(G.W4_LAYOUT_W4A16, Wq, N, K, s, z)
        nbytes = decode_bytes(M, N, K)
        C = torch.empty((M, N), dtype=torch.float16, device=dev)
        copies, warm = copies_of(Wp)
        fn = lambda i, cps=copies: G.w4a16_gemm(A, cps[i % len(cps)], N, workspace=ws, C=C)
    else:
        Aq, sa, _ = G.quantize_a8(A)
        out = G.W4_OUT_F32 if case.out == "f32" else G.W4_OUT_F16
        C = torch.empty((M, N), dtype=torch.float32 if out == G.W4_OUT_F32 else torch.float16,
                        device=dev)
        if case.scheme == "f8f8":
            Aq, sa = G.quantize_f8(A)
            Wq, wsc = G.quantize_f8(torch.from_numpy(d["W"]).to(dev))
            Wp = G.prepack_w(G.W4_LAYOUT_W8A8, Wq, N, K)
            mm, wbytes = G.f8f8_gemm, N * K + 4 * N
        elif case.scheme == "w4a8":
            Wq, wsc, _ = G.quantize_pack_w4(torch.from_numpy(d["W"]).to(dev), G.W4_SYM_PER_CHANNEL)
            Wp = G.prepack_w(G.W4_LAYOUT_W4A8, Wq, N, K)
            mm, wbytes = G.w4a8_gemm, N * K // 2 + 4 * N
        elif case.scheme == "w8a8":
            Wq, wsc = G.quantize_pack_w8(torch.from_numpy(d["W"]).to(dev))
            Wp = G.prepack_w(G.W4_LAYOUT_W8A8, Wq, N, K)
            mm, wbytes = G.w8a8_gemm, N * K + 4 * N
        else:
            Wq = G.quantize_pack_w2(torch.from_numpy(d["codes"]).to(dev))
            Wp = G.prepack_w(G.W4_LAYOUT_W2A8, Wq, N, K)
            wsc = G.ternary_scale_f16(torch.from_numpy(d["src"]).to(dev))
            mm, wbytes = G.w2a8_gemm, N * K // 4 + 2
        nbytes = wbytes + M * K + 4 * M + M * N * C.element_size()
        copies, warm = copies_of(Wp)
        fn = lambda i, cps=copies: mm(Aq, sa, cps[i % len(cps)], wsc, N, out_dtype=out,
                                      workspace=ws, C=C)
    ms = time_graph(fn, steps, warmup, stream, flush, lambda i: fn(i, warm))
    del copies, warm
    torch.cuda.empty_cache()
    return {"case": case.name, "M": M, "N": N, "K": K, "us": round(ms * 1e3, 3),
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "TOPS": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 2)}


# ---------------------------------------------------------------------------
# the oracle on the host CPU
# ---------------------------------------------------------------------------
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return platform.processor() or "unknown"


def host_cores():
    """CPU threads this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _timed_oracle(fn, threads, budget_s, max_reps):
    """Repeat fn() with the BLAS pool limited to `threads` for about
    budget_s; returns (reps, seconds)."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=threads, user_api="blas"):
        fn()                                   # first call outside the clock
        reps, t = 0, time.time()
        while True:
            fn()
            reps += 1
            el = time.time() - t
            if el > budget_s or reps >= max_reps:
                return reps, el


def cpu_baseline_decode(c, budget_s=6.0):
    """The oracle, untuned, on the host: full M=1 N=K=4096 W4A16 calls
    (dequantise in float64, then A @ W^T) with one BLAS thread and with all
    of the process's cores."""
    import oracle as O
    d = c.inputs()
    q, s, z = O.quantize_w4_group(d["W"], 128)
    fn = lambda: O.w4a16_gemm(d["A"], q, s, z, 128)
    nb = decode_bytes(c.M, c.N, c.K)
    cores = host_cores()
    out = {}
    for key, threads in (("single_thread", 1), ("all_cores", cores)):
        reps, el = _timed_oracle(fn, threads, budget_s, 200)
        out[key] = {"value": nb * reps / el / 1e9, "unit": "GB/s", "cores": threads,
                    "ms_per_call": el / reps * 1e3}
    return {"value": out["all_cores"]["value"], "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "single_thread": out["single_thread"],
            "sample": f"full oracle calls of the M=1 N=4096 K=4096 W4A16 GEMV (weights "
                      f"pre-quantised), ~{budget_s:.0f} s per thread count; all {cores} cores "
                      f"{out['all_cores']['ms_per_call']:.1f} ms/call, one thread "
                      f"{out['single_thread']['ms_per_call']:.1f} ms/call"}


def cpu_baseline_prefill(c, budget_s=6.0, rows=8):
    """The oracle on a row sample of the prefill GEMM: `rows` of the 2048
    token rows x all 11008 outputs x K=4096 (INT64 sums plus epilogue, as
    the oracle computes them), with one thread and with all cores."""
    import oracle as O
    d = c.inputs()
    q, s = O.quantize_w4_sym(d["W"])
    A = d["A"][:rows]

    def fn():
        qa, sa, _ = O.quantize_a8(A)
        O.w4a8_gemm(qa, sa, q, s, d["bias"], O.OUT_F16)

    ops = 2.0 * rows * c.N * c.K
    cores = host_cores()
    out = {}
    for key, threads in (("single_thread", 1), ("all_cores", cores)):
        reps, el = _timed_oracle(fn, threads, budget_s, 100)
        out[key] = {"value": ops * reps / el / 1e12, "unit": "TOPS", "cores": threads,
                    "ms_per_call": el / reps * 1e3}
    return {"value": out["all_cores"]["value"], "unit": "TOPS", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "single_thread": out["single_thread"],
            "sample": f"oracle calls on {rows} of {c.M} token rows (N=11008, K=4096), "
                      f"~{budget_s:.0f} s per thread count"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-prefill", action="store_true", help="skip the M=2048 GEMM")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the W4A8 M=1 context (quantize_a8 + GEMV vs the fused call)")
    ap.add_argument("--only", choices=["decode", "prefill"], default=None,
                    help="time one workload only (for profiler runs): the decode GEMV at each "
                         "of its shapes, or the prefill; prints one JSON line per shape")
    ap.add_argument("--calib", action="store_true",
                    help="also run a copy of known size (for PMC byte-counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="time every configured workload shape (graph replay); one JSON line "
                         "per case")
    ap.add_argument("--case", default=None,
                    help="with --sweep: time only the workload cases whose name contains this")
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed steps one by one from Python instead of replaying "
                         "them from one captured HIP graph")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(column/row sharding is described in the design notes, not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gemv_nibble_unpack_amd as G
    G.load()
    assert torch.cuda.is_available(), "needs a GPU"
    stream = torch.cuda.current_stream()
    flush = Flush(torch.device("cuda:0"))

    if args.sweep:
        from gemv_nibble_unpack_amd import workloads as WL
        for case in WL.ALL_CASES:
            if args.case and args.case not in case.name:
                continue
            print(json.dumps(bench_case(case, max(20, args.steps // 4), args.warmup, stream,
                                        flush)), flush=True)
        return
    if args.only == "prefill":
        cp, pre = bench_prefill(args, stream, flush)
        if args.calib:
            calibration_copy()
        ops = 2.0 * cp.M * cp.N * cp.K
        print(json.dumps({"workload": "w4a8_prefill_gemm", **pre,
                          "gemm_tops": ops / (pre["gemm_ms"] * 1e-3) / 1e12}), flush=True)
        return

    shapes = DECODE_SHAPES
    dec = []
    for (N, K) in shapes:
        log(f"bench: decode W4A16 M=1 N={N} K={K}")
        dec.append(bench_decode_shape(N, K, args.steps, args.warmup, stream, flush,
                                      eager=args.eager, probe=args.only != "decode"))
        log("bench:", {k: v for k, v in dec[-1].items() if k != "ms"})
    head = dec[0]
    if args.only == "decode":
        if args.calib:
            calibration_copy()
        for x in dec:
            print(json.dumps({"workload": "w4a16_decode_gemv", **x}), flush=True)
        return

    gbs = head["bytes"] / (head["ms"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "w4a16_decode_gemv", "M": 1, "N": 4096, "K": 4096,
                   "weights": "uint4 group128 fp16 scale + uint8 zero", "act": "fp16",
                   "out": "fp16", "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                   "cold_weight_copies": head["copies"],
                   "llc_flush_bytes": FLUSH_BYTES,
                   "cold_gap_bytes": head["cold_gap_bytes"],
                   "timing": ("eager launches" if args.eager else
                              "one HIP-graph replay of the timed steps, after an untimed replay "
                              "and a last-level-cache flush"),
                   "eager_GBps": round(head["bytes"] / (head["eager_us"] * 1e-6) / 1e9, 2)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_of(DECODE_TRAFFIC),
                     "bytes_per_launch": head["bytes"],
                     "achievable": head["achievable"],
                     "frac_of_achievable": head["frac_of_achievable"],
                     "shapes": [{**{k: v for k, v in x.items() if k not in ("ms",)},
                                 "traffic": traffic_of(decode_traffic_path(x["N"], x["K"]))}
                                for x in dec]},
        "offline_prep_ms": head["offline_prep_ms"],
    }
    if not args.no_prefill:
        log("bench: prefill W4A8 M=2048 N=11008 K=4096")
        cp, pre = bench_prefill(args, stream, flush)
        log("bench: prefill", pre)
        ops = 2.0 * cp.M * cp.N * cp.K
        tops = lambda ms: ops / (ms * 1e-3) / 1e12
        line["prefill"] = {
            "metric": "W4A8 GEMM TOPS at M=2048 (the GEMM alone; steps with activation "
                      "quantization beside it)",
            "value": round(tops(pre["gemm_ms"]), 2), "unit": "TOPS",
            "ms_per_step": round(pre["gemm_ms"], 5), "steps": pre["steps"], "dtype": "i8",
            "timing": ("eager launches" if args.eager else
                       "one HIP-graph replay per figure, after an untimed replay and a "
                       "last-level-cache flush"),
            "two_call_step": {"ms": round(pre["two_call_step_ms"], 5),
                              "TOPS": round(tops(pre["two_call_step_ms"]), 2),
                              "what": "quantize_a8 + w4a8_gemm"},
            "fused_step": {"ms": round(pre["fused_step_ms"], 5),
                           "TOPS": round(tops(pre["fused_step_ms"]), 2),
                           "what": "w4a8_gemm_fused_act (fp16 A in, one call)"},
            "quantize_a8_ms": round(pre["quant_only_ms"], 5),
            "config": {"workload": "w4a8_prefill_gemm", "M": cp.M, "N": cp.N, "K": cp.K,
                       "weights": "int4 sym per-channel", "act": "int8 per-token",
                       "out": "fp16 + bias", "cold_weight_copies": pre["copies"],
                       "cold_gap_bytes": pre["cold_gap_bytes"]},
            "roofline": {"bound": "mfma", "achieved": round(tops(pre["gemm_ms"]), 2),
                         "peak": I8_PEAK_TOPS, "unit": "TOPS",
                         "frac": round(tops(pre["gemm_ms"]) / I8_PEAK_TOPS, 4),
                         "traffic": traffic_of(PREFILL_TRAFFIC),
                         "bytes_per_launch": pre["bytes"]},
        }
    if not args.no_extra:
        log("bench: W4A8 M=1 two launches vs fused")
        line["decode_context"] = {"w4a8_m1": bench_decode_w4a8(stream, min(args.steps, 100),
                                                               flush)}
    if not args.no_cpu:
        from gemv_nibble_unpack_amd import workloads as WL
        log("bench: cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline_decode(WL.W4A16_DECODE)
        if not args.no_prefill:
            line["prefill"]["cpu_baseline"] = cpu_baseline_prefill(WL.W4A8_PREFILL)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
