"""ctypes loader for the HIP library (no torch types cross this boundary)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libgemv_nibble_unpack.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

# status codes and enumerations (mirror include/gemv_nibble_unpack.h)
W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN, W4_ERR_ARG, W4_ERR_WORKSPACE, W4_ERR_HIP = (
    0, -1, -2, -3, -4, -5, -6)
W4_ERR_SCRATCH = -7
W4_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024
W4_SYM_PER_CHANNEL, W4_ASYM_GROUP = 0, 1
W4_OUT_F16, W4_OUT_F32, W4_OUT_I32, W4_OUT_I8 = 0, 1, 2, 3
W4_IN_F16, W4_IN_F32 = 0, 1
W4_LAYOUT_W4A8, W4_LAYOUT_W4A16, W4_LAYOUT_W2A8, W4_LAYOUT_W8A8 = 0, 1, 2, 3
W4_OP_W4A8, W4_OP_W4A16, W4_OP_W2A8, W4_OP_W2A16, W4_OP_W8A8, W4_OP_F8F8 = 0, 1, 2, 3, 4, 5
W4_GROUP_SIZE = 128
W4_MAX_K = 131056

_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
_i64 = ctypes.c_int64

# name -> (restype, argtypes); the order follows the header
SIGNATURES = {
    "w4_status_string": (ctypes.c_char_p, [_i]),
    "quantize_pack_w4": (_i, [_p, _i, _i, _i, _i, _p, _p, _p, _p]),
    "quantize_pack_w2": (_i, [_p, _i, _i, _p, _p]),
    "ternary_scale_f16": (_i, [_p, _i64, _p, _p]),
    "prepack_bytes": (_sz, [_i, _i, _i]),
    "prepack_w": (_i, [_i, _p, _p, _p, _i, _i, _p, _p]),
    "unprepack_w": (_i, [_i, _p, _i, _i, _p, _p, _p, _p]),
    "quantize_a8": (_i, [_p, _i, _i, _i, _p, _p, _p, _p]),
    "w4_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "w4a8_gemm": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _p, _sz, _p]),
    "w2a8_gemm": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _p, _sz, _p]),
    "w4a16_gemm": (_i, [_p, _p, _i, _p, _p, _i, _i, _i, _p, _sz, _p]),
    "w2a16_gemm": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _p, _sz, _p]),
    "quantize_pack_w8": (_i, [_p, _i, _i, _p, _p, _p]),
    "w8a8_gemm": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _p, _sz, _p]),
    "quantize_f8": (_i, [_p, _i, _i, _i, _p, _p, _p]),
    "f8f8_gemm": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _p, _sz, _p]),
    "w4_fused_act_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "w4a8_gemm_fused_act": (_i, [_p, _i, _p, _p, _p, _p, _i, _i, _i, _i, _p, _sz, _p]),
    "w2a8_gemm_fused_act": (_i, [_p, _i, _p, _p, _p, _p, _i, _i, _i, _i, _p, _sz, _p]),
    "w4a8_gemm_fused_act_noalloc": (_i, [_p, _i, _p, _p, _p, _p, _i, _i, _i, _i, _p]),
    "w4_plan_count": (_i, [_i, _i, _i, _i]),
    "w4_plan_name": (_i, [_i, _i, _i, _i, _i, ctypes.c_char_p, _sz]),
    "w4_plan_pin": (_i, [_i, _i, _i, _i, _i]),
    "w4_plan_current": (_i, [_i, _i, _i, _i]),
    "w4_plan_reset": (_i, []),
    "w4_plan_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "w4_read_probe": (_i, [_p, _sz, _i, _p, _p]),
    "w4_graph_begin": (_i, [_p]),
    "w4_graph_end": (_i, [_p, ctypes.POINTER(_p)]),
    "w4_graph_update": (_i, [_p, _p]),
    "w4_graph_launch": (_i, [_p, _p]),
    "w4_graph_kernel_nodes": (_i, [_p]),
    "w4_graph_destroy": (_i, [_p]),
}

_LIB = None


class LibraryMissing(RuntimeError):
    """The compiled HIP library is not present; there is no fallback path."""


def load():
    """Load (once) and return the ctypes handle of the HIP library."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            f"{LIB_PATH} not found: build it first (python -c 'import __graft_entry__ as g; g.build()')"
            " -- this package has no CPU fallback")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


class W4Error(RuntimeError):
    def __init__(self, fn, status):
        text = load().w4_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def check(fn, status):
    if status != W4_OK:
        raise W4Error(fn, status)
    return status
