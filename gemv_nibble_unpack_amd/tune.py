"""Shape-keyed plan tuning on the GPU.

After the KoGPT FasterTransformer page, section 2.3 (GEMM tuning): time every
candidate plan the library offers for a shape, keep the fastest per
(op, M, N, K) in a table, and re-tune on each GPU model. The candidates
compute the same result (INT32 and INT8 outputs are identical across plans),
so pinning one only changes speed.

    from gemv_nibble_unpack_amd import tune
    table = tune.tune([(G.W4_OP_W4A8, 2048, 4096, 4096), (G.W4_OP_W4A16, 16, 4096, 4096)])
    tune.save("plans.json", table)       # later, in another process:
    tune.load("plans.json")              # pins the recorded plans by name

Timing: each candidate's calls are captured in one HIP graph (the plan is
chosen when a call is issued, so the graph holds that plan) and replayed over
rotating copies of the weights large enough to leave the last-level cache
cold, as in the benchmark.
"""
from __future__ import annotations

import json
import math

import torch

from . import _lib as L
from . import api as G
from . import workloads as WL

OPS = {"w4a8": L.W4_OP_W4A8, "w4a16": L.W4_OP_W4A16, "w2a8": L.W4_OP_W2A8,
       "w2a16": L.W4_OP_W2A16, "w8a8": L.W4_OP_W8A8, "f8f8": L.W4_OP_F8F8}
OP_NAMES = {v: k for k, v in OPS.items()}
ROTATE_BYTES = 1 << 30


def candidates(op, M, N, K):
    """Names of the shape's candidate plans, in index order."""
    return [G.w4_plan_name(op, M, N, K, i) for i in range(G.w4_plan_count(op, M, N, K))]


def _operands(op, M, N, K, device, seed):
    """Device operands for one shape and a call taking (weights, C, workspace)."""
    A = torch.from_numpy(WL.activations(M, K, seed=seed)).to(device)
    if op in (L.W4_OP_W2A8, L.W4_OP_W2A16):
        codes = torch.from_numpy(WL.ternary_codes(N, K, seed=seed + 1)).to(device)
        Wp = G.prepack_w(L.W4_LAYOUT_W2A8, G.quantize_pack_w2(codes), N, K)
        src = torch.from_numpy(WL.weights_f32(1, 1024, seed=seed + 2)).to(device)
        scale = G.ternary_scale_f16(src)
    elif op == L.W4_OP_W4A16:
        W = torch.from_numpy(WL.weights_f32(N, K, seed=seed + 1)).to(device)
        Wq, s, z = G.quantize_pack_w4(W, L.W4_ASYM_GROUP)
        Wp, scale = G.prepack_w(L.W4_LAYOUT_W4A16, Wq, N, K, s, z), None
    elif op == L.W4_OP_W8A8:
        W = torch.from_numpy(WL.weights_f32(N, K, seed=seed + 1)).to(device)
        Wq, scale = G.quantize_pack_w8(W)
        Wp = G.prepack_w(L.W4_LAYOUT_W8A8, Wq, N, K)
    elif op == L.W4_OP_F8F8:
        W = torch.from_numpy(WL.weights_f32(N, K, seed=seed + 1)).to(device)
        Wq, scale = G.quantize_f8(W)
        Wp = G.prepack_w(L.W4_LAYOUT_W8A8, Wq, N, K)
    else:
        W = torch.from_numpy(WL.weights_f32(N, K, seed=seed + 1)).to(device)
        Wq, scale, _ = G.quantize_pack_w4(W, L.W4_SYM_PER_CHANNEL)
        Wp = G.prepack_w(L.W4_LAYOUT_W4A8, Wq, N, K)
    C = torch.empty((M, N), dtype=torch.float16, device=device)
    if op == L.W4_OP_F8F8:
        Aq, sa = G.quantize_f8(A)
        call = lambda w, ws: G.f8f8_gemm(Aq, sa, w, scale, N, workspace=ws, C=C)
    elif op in (L.W4_OP_W4A8, L.W4_OP_W2A8, L.W4_OP_W8A8):
        Aq, sa, _ = G.quantize_a8(A)
        mm = {L.W4_OP_W4A8: G.w4a8_gemm, L.W4_OP_W2A8: G.w2a8_gemm, L.W4_OP_W8A8: G.w8a8_gemm}[op]
        call = lambda w, ws: mm(Aq, sa, w, scale, N, workspace=ws, C=C)
    elif op == L.W4_OP_W4A16:
        call = lambda w, ws: G.w4a16_gemm(A, w, N, workspace=ws, C=C)
    else:
        call = lambda w, ws: G.w2a16_gemm(A, w, scale, N, workspace=ws, C=C)
    return Wp, call


def _time_plan(call, copies, ws, reps, warmup):
    """Mean microseconds per call: `reps` calls over the rotating weight copies,
    captured in one graph and replayed once untimed, once timed."""
    for i in range(warmup):
        call(copies[i % len(copies)], ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            call(copies[i % len(copies)], ws)
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / reps


def tune_shape(op, M, N, K, device="cuda", reps=50, warmup=3, seed=0, pin=True):
    """Time every candidate plan of one shape; pin the fastest when ``pin``.

    Returns {"op", "M", "N", "K", "plan", "us", "candidates": {name: us}}.
    Any pin the shape had is removed while timing and replaced afterwards
    (restored when ``pin`` is false).
    """
    dev = torch.device(device)
    before = G.w4_plan_current(op, M, N, K)
    Wp, call = _operands(op, M, N, K, dev, seed)
    ncopies = min(reps, max(1, math.ceil(ROTATE_BYTES / Wp.numel())))
    copies = [Wp] + [Wp.clone() for _ in range(ncopies - 1)]
    times = {}
    try:
        for i, name in enumerate(candidates(op, M, N, K)):
            G.w4_plan_pin(op, M, N, K, i)
            need = G.w4_plan_workspace_bytes(op, M, N, K)
            # a zeroed workspace per candidate, as for any first use
            ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev) if need else None
            times[name] = _time_plan(call, copies, ws, reps, warmup)
    finally:
        G.w4_plan_pin(op, M, N, K, -1)
    best = min(times, key=times.get)
    names = list(times)
    G.w4_plan_pin(op, M, N, K, names.index(best) if pin else -1)
    if not pin and before != G.w4_plan_current(op, M, N, K):
        G.w4_plan_pin(op, M, N, K, before)
    del copies
    return {"op": OP_NAMES[op], "M": M, "N": N, "K": K, "plan": best,
            "us": round(times[best], 3), "candidates": {k: round(v, 3) for k, v in times.items()}}


def tune(shapes, **kw):
    """Tune and pin each (op, M, N, K) in ``shapes``; returns the table."""
    return [tune_shape(op, M, N, K, **kw) for op, M, N, K in shapes]


def save(path, table):
    """Write the table (op names, sizes and plan names) as JSON."""
    with open(path, "w") as f:
        json.dump({"plans": [{k: r[k] for k in ("op", "M", "N", "K", "plan", "us")} for r in table]},
                  f, indent=1)


def load(path):
    """Pin every plan recorded in a saved table, by name. Entries whose plan
    this library no longer offers for the shape are skipped and returned."""
    with open(path) as f:
        rows = json.load(f)["plans"]
    skipped = []
    for r in rows:
        op = OPS[r["op"]]
        names = candidates(op, r["M"], r["N"], r["K"])
        if r["plan"] in names:
            G.w4_plan_pin(op, r["M"], r["N"], r["K"], names.index(r["plan"]))
        else:
            skipped.append(r)
    return skipped


def workload_shapes():
    """The distinct (op, M, N, K) of the configured workload cases."""
    seen = []
    for c in WL.ALL_CASES:
        s = (OPS[c.scheme], c.M, c.N, c.K)
        if s not in seen:
            seen.append(s)
    return seen


def main(argv=None):
    """Tune the configured workload shapes; print one JSON line per shape
    (tuned plan, built-in plan, every candidate's time) and save the table."""
    import argparse
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", default=None, help="write the tuned table here (JSON)")
    ap.add_argument("--reps", type=int, default=50)
    ap.add_argument("--scheme", action="append", default=None, choices=sorted(OPS),
                    help="tune only the shapes of this weight/activation scheme (repeatable)")
    ap.add_argument("--min-m", type=int, default=1, help="tune only shapes with M >= this")
    args = ap.parse_args(argv)
    want = {OPS[k] for k in args.scheme} if args.scheme else None
    table = []
    for op, M, N, K in workload_shapes():
        if (want is not None and op not in want) or M < args.min_m:
            continue
        G.w4_plan_pin(op, M, N, K, -1)
        builtin = candidates(op, M, N, K)[G.w4_plan_current(op, M, N, K)]
        rec = tune_shape(op, M, N, K, reps=args.reps)
        rec["builtin"] = builtin
        rec["builtin_us"] = rec["candidates"][builtin]
        print(json.dumps(rec), flush=True)
        table.append(rec)
    if args.out:
        save(args.out, table)
    return table


if __name__ == "__main__":
    main()
