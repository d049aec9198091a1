"""Build the HIP library in-tree for gfx950 (cross-compiles without a GPU).

    python -m gemv_nibble_unpack_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["quant.hip", "prepack.hip", "matmul.hip", "probe.hip", "noalloc.hip"]
OUT = os.path.join(HERE, "libgemv_nibble_unpack.so")
ARCH = os.environ.get("W4_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    # correctly rounded float32 division: the quantizers decide codes with '/'
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    # no packed-FP32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument", *os.environ.get("W4_EXTRA_FLAGS", "").split(),
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose=True):
    """Compile every HIP source into the package's shared library."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = OUT + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
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
