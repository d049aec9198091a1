"""Shared helpers for the GPU parity tests (comparison rules and oracle runs)."""
from __future__ import annotations

import sys

import numpy as np

import oracle as O


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tol_ok(gpu, ref, what=""):
    """|gpu - ref| <= 2^-9 |ref| + 1e-3 rms(ref), element-wise."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(gpu - ref)
    bound = 2.0 ** -9 * np.abs(ref) + 1e-3 * rms
    bad = err > bound
    if np.any(bad):
        i = int(np.argmax(err - bound))
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{bad.size} outside tolerance; worst at flat {i}: "
            f"gpu={gpu.ravel()[i]!r} ref={ref.ravel()[i]!r} bound={bound.ravel()[i]!r}")
    return float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0


def sample_indices(M, N, count, seed):
    """Sampled (row, col) pairs: the corners, the ragged edges and random ones."""
    rng = np.random.default_rng(seed)
    rows = [0, M - 1, 0, M - 1, M // 2]
    cols = [0, 0, N - 1, N - 1, N // 2]
    rows += rng.integers(0, M, count).tolist()
    cols += rng.integers(0, N, count).tolist()
    return np.array(rows), np.array(cols)
