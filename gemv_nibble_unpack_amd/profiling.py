"""Turn rocprofv3 output into the short text summaries kept under profiles/.

    python -m gemv_nibble_unpack_amd.profiling trace <rocprof_dir> <out.md> --cmd "<command>"
    python -m gemv_nibble_unpack_amd.profiling traffic <fetch_dir> <write_dir> <out.json> \
        --kernel <substring> --calib-bytes <bytes> [--calib-kernel <substring>] --cmd "<commands>"
    python -m gemv_nibble_unpack_amd.profiling counters <out.md> <pmc_dir>... \
        --kernel <substring> [--grid <threads>] --cmd "<command>" [--cmd ...]

``trace`` reads a ``--kernel-trace --output-format csv`` directory and writes
per-kernel call counts and durations. ``traffic`` reads two ``--pmc
FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs (KiB per dispatch) of a program that
also ran a plain device-to-device copy of ``calib-bytes`` bytes; the copy's
counter readings give the scale factor from counter KiB to real bytes, and the
kernel's readings times that factor give its HBM bytes per launch. The JSON
also records a hash of the kernel sources so a later benchmark run reports the
traffic only while the kernel is unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")


def kernel_source_hash():
    """sha256 over every HIP source of the library (any change invalidates)."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def _grid(row):
    """The launch shape of a dispatch as 'grid x*y*z / block x' (threads)."""
    return (f"{row['Grid_Size_X']}x{row['Grid_Size_Y']}x{row['Grid_Size_Z']}"
            f" / {row['Workgroup_Size_X']}")


def trace_rows(d):
    """(kernel name, launch shape, duration ns) per dispatch from a
    kernel-trace CSV dir."""
    path = _find(d, "kernel_trace.csv")
    out = []
    with open(path) as f:
        for row in csv.DictReader(f):
            out.append((row["Kernel_Name"], _grid(row),
                        int(row["End_Timestamp"]) - int(row["Start_Timestamp"])))
    return out


def summarize_trace(d, out_path, cmd):
    """Per (kernel, launch shape): one product shape launches one grid, so
    the shapes of one kernel template are listed apart."""
    rows = trace_rows(d)
    by = defaultdict(list)
    for name, grid, ns in rows:
        by[(name, grid)].append(ns / 1e3)
    lines = ["# rocprofv3 kernel trace summary", "", f"Command: `{cmd}`", "",
             "| kernel | grid / block (threads) | calls | mean us | median us | min us |",
             "|---|---|---|---|---|---|"]
    for (name, grid), v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        short = name if len(name) < 90 else name[:87] + "..."
        lines.append(f"| `{short}` | {grid} | {len(v)} | {statistics.mean(v):.2f} | "
                     f"{statistics.median(v):.2f} | {min(v):.2f} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out_path


def pmc_values(d, counter, grid=None, keep="bitwise_not"):
    """Counter readings per kernel name; with ``grid`` (total threads), only
    the dispatches of that launch size, and every dispatch of the kernels
    whose name contains ``keep`` (the calibration copy)."""
    path = _find(d, "counter_collection.csv")
    out = defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            if grid is not None and int(row["Grid_Size"]) != grid and \
                    keep not in row["Kernel_Name"]:
                continue
            out[row["Kernel_Name"]].append(float(row["Counter_Value"]))
    return out


def summarize_traffic(fetch_dir, write_dir, out_path, kernel, calib_bytes, cmd,
                      calib_kernel="bitwise_not", grid=None):
    fetch = pmc_values(fetch_dir, "FETCH_SIZE", grid, calib_kernel)
    write = pmc_values(write_dir, "WRITE_SIZE", grid, calib_kernel)

    def pick(table, key):
        vals = [v for name, vs in table.items() if key in name for v in vs]
        if not vals:
            raise KeyError(f"no dispatch matching {key!r}")
        return statistics.median(vals)

    def copy_kernel(table):
        names = [n for n in table if calib_kernel in n]
        if not names:
            raise KeyError(f"no calibration kernel matching {calib_kernel!r}")
        return names[0]

    cf, cw = copy_kernel(fetch), copy_kernel(write)
    f_scale = calib_bytes / statistics.median(fetch[cf])
    w_scale = calib_bytes / statistics.median(write[cw])
    kf, kw = pick(fetch, kernel), pick(write, kernel)
    rec = {
        "kernel": kernel,
        "grid_threads": grid,
        "fetch_kib_per_launch": kf, "write_kib_per_launch": kw,
        "calibration": {"copy_kernel": cf, "bytes": calib_bytes,
                        "fetch_kib": statistics.median(fetch[cf]),
                        "write_kib": statistics.median(write[cw]),
                        "fetch_bytes_per_kib": f_scale, "write_bytes_per_kib": w_scale},
        "read_bytes_per_launch": kf * f_scale,
        "write_bytes_per_launch": kw * w_scale,
        "traffic_bytes_per_launch": kf * f_scale + kw * w_scale,
        "source_hash": kernel_source_hash(),
        "command": cmd,
    }
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def summarize_mfma(util_dir, raw_dir, out_path, kernel, ops, cmds):
    """Matrix-core evidence for one kernel from two counter passes: the derived
    MfmaUtil (busy MFMA cycles over all SIMDs / (GPU-active cycles x SIMDs)),
    and the raw I8 MFMA operation count (x 512) with the busy cycles and the
    GPU-active cycles (summed over the XCDs). Medians per launch."""
    def pick(d, counter):
        vals = [v for name, vs in pmc_values(d, counter).items() if kernel in name for v in vs]
        if not vals:
            raise KeyError(f"no {counter} for a dispatch matching {kernel!r}")
        return statistics.median(vals), len(vals)

    util, n = pick(util_dir, "MfmaUtil")
    mops, _ = pick(raw_dir, "SQ_INSTS_VALU_MFMA_MOPS_I8")
    busy, _ = pick(raw_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    active, _ = pick(raw_dir, "GRBM_GUI_ACTIVE")
    lines = ["# rocprofv3 matrix-core counters", "",
             f"Kernel: `{kernel}` ({n} launches, medians per launch)", "",
             "| quantity | value |", "|---|---|",
             f"| MfmaUtil (busy MFMA cycles / (GPU-active cycles x SIMDs)) | {util:.1f} % |",
             f"| I8 MFMA operations (SQ_INSTS_VALU_MFMA_MOPS_I8 x 512) | {mops * 512:.4e} |",
             f"| algorithmic operations 2*M*N*K | {ops:.4e} |",
             f"| executed / algorithmic (padding of the last block's columns) | {mops * 512 / ops:.4f} |",
             f"| SQ_VALU_MFMA_BUSY_CYCLES (all SIMDs) | {busy:.0f} |",
             f"| GRBM_GUI_ACTIVE (summed over the XCDs) | {active:.0f} |",
             "", "Commands:", ""] + [f"* `{c}`" for c in cmds]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out_path


def summarize_counters(dirs, out_path, kernel, cmds, grid=None):
    """Every counter of one or more ``--pmc`` passes for the dispatches of one
    kernel (name substring) and, with ``grid``, one launch size: the median
    per launch, and per wave where the pass also counted SQ_WAVES."""
    per = {}
    n = 0
    for d in dirs:
        path = _find(d, "counter_collection.csv")
        vals = defaultdict(list)
        with open(path) as f:
            for row in csv.DictReader(f):
                if kernel not in row["Kernel_Name"]:
                    continue
                if grid is not None and int(row["Grid_Size"]) != grid:
                    continue
                vals[row["Counter_Name"]].append(float(row["Counter_Value"]))
        if not vals:
            raise KeyError(f"no dispatch matching {kernel!r} in {d}")
        n = max(n, max(len(v) for v in vals.values()))
        per.update({c: statistics.median(v) for c, v in vals.items()})
    waves = per.get("SQ_WAVES")
    lines = ["# rocprofv3 counters", "",
             f"Kernel: `{kernel}`" + (f", {grid} threads per launch" if grid else "") +
             f" ({n} launches, medians per launch)", "",
             "| counter | per launch | per wave |", "|---|---|---|"]
    for c in sorted(per):
        pw = f"{per[c] / waves:.1f}" if waves else ""
        lines.append(f"| {c} | {per[c]:.0f} | {pw} |")
    if "SQ_LDS_BANK_CONFLICT" in per and per.get("SQ_ACTIVE_INST_LDS"):
        lines += ["", f"LDS bank-conflict cycles / LDS-active cycles: "
                      f"{per['SQ_LDS_BANK_CONFLICT'] / per['SQ_ACTIVE_INST_LDS']:.2f}"]
    lines += ["", "Commands:", ""] + [f"* `{c}`" for c in cmds]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return per


def load_traffic(path):
    """The recorded traffic, or None if absent or the kernels changed since."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("out")
    t.add_argument("--cmd", required=True)
    q = sub.add_parser("traffic")
    q.add_argument("fetch_dir")
    q.add_argument("write_dir")
    q.add_argument("out")
    q.add_argument("--kernel", required=True)
    q.add_argument("--calib-bytes", type=int, required=True)
    q.add_argument("--calib-kernel", default="bitwise_not",
                   help="name substring of the calibration copy kernel")
    q.add_argument("--grid", type=int, default=None,
                   help="only dispatches of this many threads (one product shape)")
    q.add_argument("--cmd", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("util_dir")
    m.add_argument("raw_dir")
    m.add_argument("out")
    m.add_argument("--kernel", required=True)
    m.add_argument("--ops", type=float, required=True, help="algorithmic operations per launch")
    m.add_argument("--cmd", action="append", required=True)
    c = sub.add_parser("counters")
    c.add_argument("out")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--grid", type=int, default=None)
    c.add_argument("--cmd", action="append", required=True)
    a = ap.parse_args()
    if a.what == "counters":
        print(json.dumps(summarize_counters(a.dirs, a.out, a.kernel, a.cmd, a.grid), indent=1))
        return
    if a.what == "mfma":
        print(summarize_mfma(a.util_dir, a.raw_dir, a.out, a.kernel, a.ops, a.cmd))
        return
    if a.what == "trace":
        print(summarize_trace(a.dir, a.out, a.cmd))
    else:
        print(json.dumps(summarize_traffic(a.fetch_dir, a.write_dir, a.out, a.kernel,
                                           a.calib_bytes, a.cmd, a.calib_kernel, a.grid),
                         indent=1))


if __name__ == "__main__":
    main()
