#!/usr/bin/env python3
"""Benchmark of the low-bit-weight matmul hot path on one MI355X.

One JSON line on stdout. Headline (``value``): the W4A16 decode GEMV at M=1,
N=K=4096 (group-128 uINT4 weights, fp16 activations, fp16 output) in GB/s of
algorithmic bytes. The same line carries the W4A8 prefill GEMM (M=2048,
N=11008, K=4096) in TOPS under ``prefill``. Every timed step reads its weights
from a different copy (>= 1 GiB of copies in rotation) so each launch streams
them from HBM, not from the 256 MB last-level cache.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-prefill]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4 GEMV HBM GB/s (% peak) at M=1; W4A8 GEMM TOPS (% MFMA peak) at M=2048"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
I8_PEAK_TOPS = 5000.0          # MI355X dense INT8 MFMA
ROTATE_BYTES = 1 << 30         # weight copies in rotation per workload
CALIB_BYTES = 256 << 20        # device-to-device copy used to calibrate PMC byte counters
PROFILES = os.path.join(ROOT, "profiles")
DECODE_TRAFFIC = os.path.join(PROFILES, "k_gemv_w4a16_decode_m1_n4096_k4096_traffic.json")
PREFILL_TRAFFIC = os.path.join(PROFILES, "k_gemm_w4a8_prefill_m2048_n11008_k4096_traffic.json")


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


def time_loop(fn, steps, warmup, stream):
    """Warm up, then time `steps` calls with events on `stream`.

    Returns (ms per step over the whole timed region, list of per-call ms
    from per-call event pairs measured in a second pass)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        fn(warmup + i)
    t1.record(stream)
    torch.cuda.synchronize()
    region_ms = t0.elapsed_time(t1) / steps
    # per-call brackets (kernel time plus event-marker overhead)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(warmup + steps + i)
        b.record(stream)
    torch.cuda.synchronize()
    per_call = [a.elapsed_time(b) for a, b in evs]
    return region_ms, per_call


def time_graph(fn, steps, warmup, stream):
    """Capture `steps` calls in one HIP graph, replay it once untimed and once
    timed; returns (ms per call, per-call list from the eager pass)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, []


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


def bench_decode(args, stream):
    import torch
    import gemv_nibble_unpack_amd as G
    from gemv_nibble_unpack_amd import workloads as WL

    c = WL.W4A16_DECODE
    d = c.inputs()
    dev = torch.device("cuda:0")
    W = torch.from_numpy(d["W"]).to(dev)
    A = torch.from_numpy(d["A"]).to(dev)
    t = time.time()
    Wq, s, z = G.quantize_pack_w4(W, G.W4_ASYM_GROUP)
    Wp = G.prepack_w(G.W4_LAYOUT_W4A16, Wq, c.N, c.K, s, z)
    torch.cuda.synchronize()
    prep_ms = (time.time() - t) * 1e3
    R = max(1, math.ceil(ROTATE_BYTES / Wp.numel()))
    copies = [Wp] + [Wp.clone() for _ in range(R - 1)]
    C = torch.empty((c.M, c.N), dtype=torch.float16, device=dev)
    ws = G.Workspace(dev)

    def step(i):
        # stream=None: the current stream (the capture stream under --graph)
        G.w4a16_gemm(A, copies[i % R], c.N, workspace=ws, C=C,
                     stream=None if not args.eager else stream)

    eager_ms, per_call = time_loop(step, args.steps, args.warmup, stream) if args.eager else \
        time_loop(lambda i: G.w4a16_gemm(A, copies[i % R], c.N, workspace=ws, C=C, stream=stream),
                  args.steps, args.warmup, stream)
    region_ms = eager_ms if args.eager else time_graph(step, args.steps, args.warmup, stream)[0]
    nbytes = decode_bytes(c.M, c.N, c.K)
    kern_ms = float(np.median(per_call))
    out = {
        "region_ms": region_ms, "eager_region_ms": eager_ms, "graph": not args.eager,
        "per_call_median_ms": kern_ms,
        "per_call_mean_ms": float(np.mean(per_call)), "bytes": nbytes, "copies": R,
        "offline_prep_ms": prep_ms,
    }
    del copies
    torch.cuda.empty_cache()
    return c, out


def bench_prefill(args, stream):
    import torch
    import gemv_nibble_unpack_amd as G
    from gemv_nibble_unpack_amd import workloads as WL

    c = WL.W4A8_PREFILL
    d = c.inputs()
    dev = torch.device("cuda:0")
    W = torch.from_numpy(d["W"]).to(dev)
    A = torch.from_numpy(d["A"]).to(dev)
    bias = torch.from_numpy(d["bias"]).to(dev)
    Wq, ws_, _ = G.quantize_pack_w4(W, G.W4_SYM_PER_CHANNEL)
    Wp = G.prepack_w(G.W4_LAYOUT_W4A8, Wq, c.N, c.K)
    del W, Wq
    R = max(1, math.ceil(ROTATE_BYTES / Wp.numel()))
    copies = [Wp] + [Wp.clone() for _ in range(R - 1)]
    Aq = torch.empty((c.M, c.K), dtype=torch.int8, device=dev)
    sa = torch.empty(c.M, dtype=torch.float32, device=dev)
    C = torch.empty((c.M, c.N), dtype=torch.float16, device=dev)
    wsp = G.Workspace(dev)
    steps = max(1, args.steps // 4)

    def step(i, st=stream):
        G.quantize_a8(A, with_rowsum=False, out=(Aq, sa, None), stream=st)
        G.w4a8_gemm(Aq, sa, copies[i % R], ws_, c.N, bias=bias, out_dtype=G.W4_OUT_F16,
                    workspace=wsp, C=C, stream=st)

    def gemm_only(i):
        G.w4a8_gemm(Aq, sa, copies[i % R], ws_, c.N, bias=bias, out_dtype=G.W4_OUT_F16,
                    workspace=wsp, C=C, stream=stream)

    eager_step_ms, _ = time_loop(step, steps, max(1, args.warmup // 4), stream)
    # the two launches of a step replayed from one captured graph (stream=None:
    # the capture stream), as the decode steps are; eager for --eager
    region_ms = eager_step_ms if args.eager else \
        time_graph(lambda i: step(i, None), steps, max(1, args.warmup // 4), stream)[0]
    gemm_ms, per_call = time_loop(gemm_only, steps, 1, stream)
    del copies
    torch.cuda.empty_cache()
    return c, {"step_ms": region_ms, "eager_step_ms": eager_step_ms, "gemm_region_ms": gemm_ms,
               "gemm_per_call_median_ms": float(np.median(per_call)), "steps": steps,
               "bytes": prefill_bytes(c.M, c.N, c.K), "copies": R}


def bench_decode_extra(stream, steps):
    """Context lines at M=1 (graph replay, cold weight copies): the W4A16
    GEMV at the two 11008-sized projection shapes, and the W4A8 GEMV with
    activations quantized by a separate kernel versus in the GEMV prologue
    (w4a8_gemm_fused_act)."""
    import torch
    import gemv_nibble_unpack_amd as G
    from gemv_nibble_unpack_amd import workloads as WL
    dev = torch.device("cuda:0")
    out = {"w4a16_m1": []}
    for c in WL.W4A16_SWEEP:
        if c.M != 1 or c.N * c.K == 4096 * 4096:
            continue
        d = c.inputs()
        Wq, s, z = G.quantize_pack_w4(torch.from_numpy(d["W"]).to(dev), G.W4_ASYM_GROUP)
        Wp = G.prepack_w(G.W4_LAYOUT_W4A16, Wq, c.N, c.K, s, z)
        del Wq
        A = torch.from_numpy(d["A"]).to(dev)
        R = max(1, math.ceil(ROTATE_BYTES / Wp.numel()))
        copies = [Wp] + [Wp.clone() for _ in range(R - 1)]
        C = torch.empty((c.M, c.N), dtype=torch.float16, device=dev)
        ws = G.Workspace(dev)
        ms, _ = time_graph(lambda i: G.w4a16_gemm(A, copies[i % R], c.N, workspace=ws, C=C),
                           steps, 10, stream)
        nb = decode_bytes(c.M, c.N, c.K)
        out["w4a16_m1"].append({"N": c.N, "K": c.K, "us": round(ms * 1e3, 3),
                                "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                                "pct_hbm_peak": round(100 * nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)})
        del copies
    # W4A8 M=1 N=K=4096: two launches vs the fused prologue
    N = K = 4096
    rng = np.random.default_rng(700)
    W = torch.from_numpy(rng.normal(0, 0.02, (N, K)).astype(np.float32)).to(dev)
    A = torch.from_numpy(rng.normal(0, 1, (1, K)).astype(np.float16)).to(dev)
    Wq, wsc, _ = G.quantize_pack_w4(W, G.W4_SYM_PER_CHANNEL)
    Wp = G.prepack_w(G.W4_LAYOUT_W4A8, Wq, N, K)
    del W, Wq
    R = max(1, math.ceil(ROTATE_BYTES / Wp.numel()))
    copies = [Wp] + [Wp.clone() for _ in range(R - 1)]
    C = torch.empty((1, N), dtype=torch.float16, device=dev)
    q = (torch.empty((1, K), dtype=torch.int8, device=dev), torch.empty(1, device=dev), None)
    ws = G.Workspace(dev)

    def two(i):
        G.quantize_a8(A, out=q)
        G.w4a8_gemm(q[0], q[1], copies[i % R], wsc, N, workspace=ws, C=C)

    def fused(i):
        G.w4a8_gemm_fused_act(A, copies[i % R], wsc, N, workspace=ws, C=C)

    nb = N * K // 2 + 4 * N + 2 * K + 2 * N
    row = {"N": N, "K": K, "bytes": nb}
    for name, fn in (("two_launch", two), ("fused", fused)):
        ms, _ = time_graph(fn, steps, 10, stream)
        row[name] = {"us": round(ms * 1e3, 3), "GBps": round(nb / (ms * 1e-3) / 1e9, 1)}
    out["w4a8_m1"] = row
    del copies
    torch.cuda.empty_cache()
    return out


def traffic_of(path):
    """HBM bytes per launch from the committed PMC summary, or None when the
    summary is missing or the kernel sources changed since it was taken."""
    from gemv_nibble_unpack_amd.profiling import load_traffic
    rec = load_traffic(path)
    return None if rec is None else round(rec["traffic_bytes_per_launch"])


def bench_case(case, steps, warmup, stream):
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
        copies = [Wp] + [Wp.clone() for _ in range(max(1, math.ceil(ROTATE_BYTES / Wp.numel())) - 1)]
        fn = lambda i: G.w2a16_gemm(A, copies[i % len(copies)], wsc, N, workspace=ws, C=C)
    elif case.scheme == "w4a16":
        Wq, s, z = G.quantize_pack_w4(torch.from_numpy(d["W"]).to(dev), G.W4_ASYM_GROUP)
        Wp = G.prepack_w(G.W4_LAYOUT_W4A16, Wq, N, K, s, z)
        nbytes = decode_bytes(M, N, K)
        C = torch.empty((M, N), dtype=torch.float16, device=dev)
        copies = [Wp] + [Wp.clone() for _ in range(max(1, math.ceil(ROTATE_BYTES / Wp.numel())) - 1)]
        fn = lambda i: G.w4a16_gemm(A, copies[i % len(copies)], N, workspace=ws, C=C)
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
        copies = [Wp] + [Wp.clone() for _ in range(max(1, math.ceil(ROTATE_BYTES / Wp.numel())) - 1)]
        fn = lambda i: mm(Aq, sa, copies[i % len(copies)], wsc, N, out_dtype=out, workspace=ws,
                          C=C)
    # the calls use the current stream: the capture stream while capturing
    ms, _ = time_graph(fn, steps, warmup, stream)
    del copies
    torch.cuda.empty_cache()
    return {"case": case.name, "M": M, "N": N, "K": K, "us": round(ms * 1e3, 3),
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "TOPS": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 2)}


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline_decode(c):
    """The oracle, untuned, on the host: full M=1 N=K=4096 W4A16 calls
    (dequantise in float64, then A @ W^T), repeated for about 10 s."""
    import oracle as O
    d = c.inputs()
    q, s, z = O.quantize_w4_group(d["W"], 128)
    reps, t = 0, time.time()
    while True:
        O.w4a16_gemm(d["A"], q, s, z, 128)
        reps += 1
        el = time.time() - t
        if el > 10.0 or reps >= 200:
            break
    gbs = decode_bytes(c.M, c.N, c.K) * reps / el / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{reps} full oracle calls of the M=1 N=4096 K=4096 W4A16 GEMV "
                      f"(weights pre-quantised) in {el:.1f} s"}


def cpu_baseline_prefill(c):
    """The oracle on a row sample of the prefill GEMM: 8 token rows x all
    11008 outputs x K=4096, INT64 accumulate plus epilogue, for about 10 s."""
    import oracle as O
    d = c.inputs()
    q, s = O.quantize_w4_sym(d["W"])
    rows = 8
    A = d["A"][:rows]
    reps, t = 0, time.time()
    while True:
        qa, sa, _ = O.quantize_a8(A)
        O.w4a8_gemm(qa, sa, q, s, d["bias"], O.OUT_F16)
        reps += 1
        el = time.time() - t
        if el > 10.0 or reps >= 100:
            break
    tops = 2.0 * rows * c.N * c.K * reps / el / 1e12
    return {"value": tops, "unit": "TOPS", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{reps} oracle calls on {rows} of {c.M} token rows (N=11008, K=4096) "
                      f"in {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-prefill", action="store_true", help="skip the M=2048 GEMM")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the M=1 context shapes (11008-sized W4A16, fused W4A8)")
    ap.add_argument("--only", choices=["decode", "prefill"], default=None,
                    help="time one workload only (for profiler runs); prints its own JSON line")
    ap.add_argument("--calib", action="store_true",
                    help="also run a copy of known size (for PMC byte-counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="time every configured workload shape (graph replay); one JSON line "
                         "per case")
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed decode steps one by one from Python instead of "
                         "replaying them from one captured HIP graph")
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

    if args.sweep:
        from gemv_nibble_unpack_amd import workloads as WL
        for case in WL.ALL_CASES:
            print(json.dumps(bench_case(case, max(20, args.steps // 4), args.warmup, stream)),
                  flush=True)
        return
    if args.only == "prefill":
        cp, pre = bench_prefill(args, stream)
        if args.calib:
            calibration_copy()
        ops = 2.0 * cp.M * cp.N * cp.K
        print(json.dumps({"workload": "w4a8_prefill_gemm", **pre,
                          "gemm_tops": ops / (pre["gemm_region_ms"] * 1e-3) / 1e12}), flush=True)
        return
    log("bench: decode W4A16 M=1 N=4096 K=4096")
    c, dec = bench_decode(args, stream)
    if args.only == "decode":
        if args.calib:
            calibration_copy()
        print(json.dumps({"workload": "w4a16_decode_gemv", **dec,
                          "gbs": dec["bytes"] / (dec["region_ms"] * 1e-3) / 1e9}), flush=True)
        return
    log("bench: decode", dec)
    gbs = dec["bytes"] / (dec["region_ms"] * 1e-3) / 1e9
    kern_gbs = dec["bytes"] / (dec["per_call_median_ms"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["region_ms"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "w4a16_decode_gemv", "M": c.M, "N": c.N, "K": c.K,
                   "weights": "uint4 group128 fp16 scale + uint8 zero", "act": "fp16",
                   "out": "fp16", "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                   "cold_weight_copies": dec["copies"],
                   "timing": "HIP-graph replay of the timed steps" if dec["graph"] else "eager",
                   "eager_GBps": round(dec["bytes"] / (dec["eager_region_ms"] * 1e-3) / 1e9, 2)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_of(DECODE_TRAFFIC),
                     "bytes_per_launch": dec["bytes"],
                     "per_call_event_gbs": round(kern_gbs, 2)},
        "offline_prep_ms": round(dec["offline_prep_ms"], 3),
    }
    if not args.no_prefill:
        log("bench: prefill W4A8 M=2048 N=11008 K=4096")
        cp, pre = bench_prefill(args, stream)
        log("bench: prefill", pre)
        ops = 2.0 * cp.M * cp.N * cp.K
        step_tops = ops / (pre["step_ms"] * 1e-3) / 1e12
        gemm_tops = ops / (pre["gemm_region_ms"] * 1e-3) / 1e12
        line["prefill"] = {
            "metric": "W4A8 GEMM TOPS at M=2048 (quantize_a8 + w4a8_gemm per step)",
            "value": round(step_tops, 2), "unit": "TOPS", "ms_per_step": round(pre["step_ms"], 5),
            "steps": pre["steps"], "dtype": "i8",
            "timing": "HIP-graph replay of the timed steps" if not args.eager else "eager",
            "eager_ms_per_step": round(pre["eager_step_ms"], 5),
            "config": {"workload": "w4a8_prefill_gemm", "M": cp.M, "N": cp.N, "K": cp.K,
                       "weights": "int4 sym per-channel", "act": "int8 per-token",
                       "out": "fp16 + bias", "cold_weight_copies": pre["copies"]},
            "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2),
                         "peak": I8_PEAK_TOPS, "unit": "TFLOP/s",
                         "frac": round(gemm_tops / I8_PEAK_TOPS, 4),
                         "traffic": traffic_of(PREFILL_TRAFFIC),
                         "gemm_ms": round(pre["gemm_region_ms"], 5)},
        }
    if not args.no_extra:
        log("bench: decode context shapes")
        line["decode_context"] = bench_decode_extra(stream, min(args.steps, 100))
    if not args.no_cpu:
        log("bench: cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline_decode(c)
        if not args.no_prefill:
            line["prefill"]["cpu_baseline"] = cpu_baseline_prefill(WL_prefill())
    print(json.dumps(line), flush=True)


def WL_prefill():
    from gemv_nibble_unpack_amd import workloads as WL
    return WL.W4A8_PREFILL


if __name__ == "__main__":
    main()
