"""Seeded synthetic inputs for the low-bit matmul workloads.

This module only draws random numbers with fixed seeds and describes the
shapes; it holds none of the quantisation or matmul arithmetic. The HIP
library's tests, the benchmark and the CPU oracle all take their inputs
from here, so both sides see the same bytes.

Distributions (the pages name model families only; shapes are the usual
LLM projection shapes):

* weights: float32 ~ N(0, 0.02)  (std-dev 0.02)
* activations: ~ N(0, 1), as float32 (W4A8 GEMV case) or float16
* bias: float16 ~ N(0, 0.01)
* ternary codes: int8 i.i.d. uniform over {-1, 0, 1}; the per-tensor scale
  comes from a separate float32 ~ N(0, 0.02) source tensor of the same shape.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WEIGHT_SIGMA = 0.02
BIAS_SIGMA = 0.01


def _rng(seed):
    return np.random.default_rng(seed)


def weights_f32(N, K, seed, sigma=WEIGHT_SIGMA):
    """float32 [N,K] ~ N(0, sigma)."""
    return (_rng(seed).standard_normal((N, K), dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def activations(M, K, seed, dtype=np.float16):
    """[M,K] ~ N(0,1) in ``dtype`` (float16 rounds the draw to nearest)."""
    return _rng(seed).standard_normal((M, K), dtype=np.float32).astype(dtype)


def bias_f16(N, seed, sigma=BIAS_SIGMA):
    """float16 [N] ~ N(0, sigma)."""
    return (_rng(seed).standard_normal(N, dtype=np.float32) * np.float32(sigma)).astype(np.float16)


def ternary_codes(N, K, seed):
    """int8 [N,K] i.i.d. uniform over {-1, 0, 1} (P(0) = 1/3)."""
    return (_rng(seed).integers(0, 3, size=(N, K), dtype=np.int8) - 1).astype(np.int8)


@dataclass(frozen=True)
class Case:
    """One (scheme, M, N, K) workload with its seeds."""
    name: str
    scheme: str          # "w4a8", "w4a16", "w2a8", "w2a16", "w8a8", "f8f8"
    M: int
    N: int
    K: int
    out: str = "f16"     # "f16", "f32", "i32"
    bias: bool = False
    act_dtype: str = "f16"
    seed: int = 0
    meta: dict = field(default_factory=dict, compare=False)

    def inputs(self):
        """Draw this case's raw inputs (before any quantisation)."""
        s = self.seed
        d = {"A": activations(self.M, self.K, s + 1,
                              np.float32 if self.act_dtype == "f32" else np.float16)}
        if self.scheme in ("w2a8", "w2a16"):
            d["codes"] = ternary_codes(self.N, self.K, s + 2)
            d["src"] = weights_f32(self.N, self.K, s + 3)
        else:
            d["W"] = weights_f32(self.N, self.K, s + 2)
        if self.bias:
            d["bias"] = bias_f16(self.N, s + 4)
        return d


def _sweep():
    out = []
    for M in (1, 4, 16):
        for (N, K) in ((4096, 4096), (11008, 4096), (4096, 11008)):
            out.append(Case(f"w4a16_sweep_M{M}_N{N}_K{K}", "w4a16", M, N, K,
                            seed=300 + 10 * M + (N // 1000) + 7 * (K // 1000)))
    return out


def _ternary():
    out = []
    for M in (1, 128):
        for (N, K) in ((3200, 3200), (8640, 3200), (3200, 8640)):
            out.append(Case(f"w2a8_M{M}_N{N}_K{K}", "w2a8", M, N, K,
                            seed=500 + M + (N // 100) + 3 * (K // 100)))
    return out


# The five workload families, in order.
W4A8_TINY = Case("w4a8_gemv_tiny", "w4a8", 1, 256, 256, out="f32", act_dtype="f32", seed=100)
W4A16_DECODE = Case("w4a16_decode_4096", "w4a16", 1, 4096, 4096, seed=200)
W4A16_SWEEP = _sweep()
W4A8_PREFILL = Case("w4a8_prefill_2048x11008x4096", "w4a8", 2048, 11008, 4096,
                    bias=True, seed=400)
W2A8_TERNARY = _ternary()

# The data-type table's FP16 x INT2 row on the same ternary weights (fp16
# activations instead of INT8), a "next" row beyond the five families.
def _ternary_a16():
    out = []
    for M in (1, 128):
        for (N, K) in ((3200, 3200), (8640, 3200), (3200, 8640)):
            out.append(Case(f"w2a16_M{M}_N{N}_K{K}", "w2a16", M, N, K,
                            seed=800 + M + (N // 100) + 3 * (K // 100)))
    return out


W2A16_TERNARY = _ternary_a16()

# The table's INT8 x INT8 row (INT8 weights with the page's /127 formula,
# INT8 per-token activations) on the 4096 x 4096 projection, M in {1, 16, 128,
# 2048}.
W8A8_CASES = [Case(f"w8a8_M{M}_N4096_K4096", "w8a8", M, 4096, 4096, seed=900 + M)
              for M in (1, 16, 128, 2048)]

# The table's FP8_E4M3 x FP8_E4M3 row (per-row E4M3 quantization of the same
# float32 weights and fp16 activations) on the 4096 x 4096 projection, M in
# {1, 16, 128, 2048}.
F8F8_CASES = [Case(f"f8f8_M{M}_N4096_K4096", "f8f8", M, 4096, 4096, seed=950 + M)
              for M in (1, 16, 128, 2048)]

# The fp16-activation prefill: W4A16 at the prefill GEMM's shape, on the tiled
# fp16 matrix-core GEMM (the 4-bit codes widened to fp16 instead of INT8; the
# FP16 x INT4 row of the BitBLAS page's data-type table), a case beyond the
# five workload families.
W4A16_PREFILL = Case("w4a16_prefill_2048x11008x4096", "w4a16", 2048, 11008, 4096,
                     bias=True, seed=450)

# The example configuration printed on the BitBLAS page (M=1, N=2048,
# K=1024, fp16 x int4, layout nt, no bias), as an extra small shape.
BITBLAS_EXAMPLE = Case("w4a16_bitblas_example", "w4a16", 1, 2048, 1024, seed=600)

ALL_CASES = [W4A8_TINY, W4A16_DECODE, *W4A16_SWEEP, W4A8_PREFILL, *W2A8_TERNARY,
             BITBLAS_EXAMPLE, *W2A16_TERNARY, *W8A8_CASES, *F8F8_CASES, W4A16_PREFILL]
