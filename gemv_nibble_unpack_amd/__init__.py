"""MI355X (gfx950) low-bit-weight matmul: C[M,N] = A[M,K] x W[N,K]^T.

A thin binding over the C ABI in ``include/gemv_nibble_unpack.h``: every
function here has the name of the C entry point it calls, takes torch device
tensors, allocates its outputs with torch (device memory and streams are all
torch is used for) and passes raw pointers and sizes down. All arithmetic runs
in the HIP kernels; if the compiled library is missing the calls raise
``LibraryMissing`` -- there is no CPU fallback.
"""
from __future__ import annotations

from ._lib import (LibraryMissing, W4Error, W4_ASYM_GROUP, W4_GROUP_SIZE, W4_IN_F16, W4_IN_F32,
                   W4_LAYOUT_W2A8, W4_LAYOUT_W4A8, W4_LAYOUT_W4A16, W4_LAYOUT_W8A8, W4_MAX_K,
                   W4_OP_F8F8, W4_OP_W2A8, W4_OP_W2A16, W4_OP_W4A8, W4_OP_W4A16, W4_OP_W8A8,
                   W4_OUT_F16,
                   W4_OUT_F32, W4_OUT_I8, W4_OUT_I32, W4_SYM_PER_CHANNEL, W4_ERR_SCRATCH,
                   W4_NOALLOC_SCRATCH_BYTES, load)
from .api import (prepack_bytes, prepack_w, quantize_a8, quantize_pack_w2, quantize_pack_w4,
                  ternary_scale_f16, unprepack_w, w2a8_gemm, w2a8_gemm_fused_act, w2a16_gemm,
                  quantize_pack_w8, w8a8_gemm, quantize_f8, f8f8_gemm,
                  w4_fused_act_workspace_bytes, w4_workspace_bytes, w4a8_gemm,
                  w4a8_gemm_fused_act, w4a16_gemm, w4_plan_count, w4_plan_current,
                  w4_plan_name, w4_plan_pin, w4_plan_reset, w4_plan_workspace_bytes, Workspace,
                  w4_read_probe, w4a8_gemm_fused_act_noalloc, StepGraph)

__all__ = [
    "LibraryMissing", "W4Error", "load", "Workspace",
    "quantize_pack_w4", "quantize_pack_w2", "ternary_scale_f16", "prepack_bytes", "prepack_w",
    "unprepack_w", "quantize_a8", "w4_workspace_bytes", "w4a8_gemm", "w2a8_gemm", "w4a16_gemm",
    "w4_fused_act_workspace_bytes", "w4a8_gemm_fused_act", "w2a8_gemm_fused_act", "w2a16_gemm",
    "quantize_pack_w8", "w8a8_gemm", "W4_OUT_I8", "W4_LAYOUT_W8A8",
    "W4_SYM_PER_CHANNEL", "W4_ASYM_GROUP", "W4_OUT_F16", "W4_OUT_F32", "W4_OUT_I32",
    "W4_IN_F16", "W4_IN_F32", "W4_LAYOUT_W4A8", "W4_LAYOUT_W4A16", "W4_LAYOUT_W2A8",
    "W4_GROUP_SIZE", "W4_MAX_K", "W4_ERR_SCRATCH", "W4_NOALLOC_SCRATCH_BYTES",
    "w4_plan_count", "w4_plan_name", "w4_plan_pin", "w4_plan_current", "w4_plan_reset",
    "w4_plan_workspace_bytes",
    "W4_OP_W4A8", "W4_OP_W4A16", "W4_OP_W2A8", "W4_OP_W2A16", "W4_OP_W8A8", "W4_OP_F8F8",
    "quantize_f8", "f8f8_gemm", "w4_read_probe", "w4a8_gemm_fused_act_noalloc", "StepGraph",
]
