"""Build the HIP library in-tree for gfx950 (cross-compiles without a GPU).

    python -m gemv_nibble_unpack_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["quant.hip", "prepack.hip", "matmul.hip", "gemm_launch.hip", "probe.hip", "noalloc.hip",
           "graph.hip", "gemm16.hip"]
OUT = os.path.join(HERE, "libgemv_nibble_unpack.so")
OBJ_DIR = os.path.join(HERE, "_build")
ARCH = os.environ.get("W4_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    # correctly rounded float32 division: the quantizers decide codes with '/'
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    # no packed-FP32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments arrive preloaded in SGPRs (up to the
    # user-SGPR limit) instead of through a kernel-argument fetch
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-command-line-argument", *os.environ.get("W4_EXTRA_FLAGS", "").split(),
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose=True, jobs=None):
    """Compile every HIP source (in parallel, one object each) and link the
    package's shared library. Each translation unit carries its own device
    code; no device function is called across units."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = [os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cflags = [f for f in FLAGS if f != "-shared"]
    cmds = [[hipcc(), *cflags, *inc, "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = OUT + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    undefined_kernels(tmp)
    os.replace(tmp, OUT)
    return OUT


def undefined_kernels(path):
    """Fail if the library references a kernel it does not define: clang drops
    a kernel's host stub without an error when the host pass cannot
    instantiate it, which would only surface when the library is loaded."""
    nm = shutil.which("nm") or "/usr/bin/nm"
    if not os.path.exists(nm):
        return
    res = subprocess.run([nm, "-C", "--undefined-only", path], capture_output=True, text=True)
    bad = [l.strip() for l in res.stdout.splitlines() if "w4::" in l]
    if bad:
        raise RuntimeError("kernels referenced but not defined:\n" + "\n".join(bad))


if __name__ == "__main__":
    print(build())
