"""Plain CPU oracle for the low-bit-weight matmul C[M,N] = A[M,K] x W[N,K]^T.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package. The product (``gemv_nibble_unpack_amd``) never imports it and
never falls back to it; the oracle in turn imports nothing from the product.

Every function is written from the pages' definitions, in their order, with
numpy as the only library (integer work in int64, floating-point references
in float64; quantisation decisions in float32 because that is the precision
the kernels take them in). See ``w4_oracle`` for the citations and for the
one function whose parity is unpinned.
"""
from .w4_oracle import *  # noqa: F401,F403
from .w4_oracle import __all__  # noqa: F401
