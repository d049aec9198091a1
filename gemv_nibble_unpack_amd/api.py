"""torch-tensor wrappers with the C entry points' names (marshalling only)."""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t):
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.device


class Workspace:
    """A zero-filled device workspace that grows on demand.

    The matmul kernels leave the part they rely on zero after each call, so
    one workspace serves any number of calls issued on one stream.
    """

    def __init__(self, device=None):
        self.device = torch.device(device or "cuda")
        self.buf = None

    def get(self, nbytes):
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


def quantize_pack_w4(W, scheme=L.W4_SYM_PER_CHANNEL, group_size=None, stream=None):
    """float32 [N,K] -> (Wq uint8 [N,K/2], scales, zeros-or-None)."""
    dev = _dev(W)
    N, K = W.shape
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    if scheme == L.W4_SYM_PER_CHANNEL:
        gs = -1 if group_size is None else group_size
        scales = torch.empty(N, dtype=torch.float32, device=dev)
        zeros = None
    else:
        gs = L.W4_GROUP_SIZE if group_size is None else group_size
        G = K // L.W4_GROUP_SIZE
        scales = torch.empty((N, G), dtype=torch.float16, device=dev)
        zeros = torch.empty((N, G), dtype=torch.uint8, device=dev)
    L.check("quantize_pack_w4", L.load().quantize_pack_w4(
        _ptr(W), N, K, scheme, gs, _ptr(Wq), _ptr(scales), _ptr(zeros), _stream(stream)))
    return Wq, scales, zeros


def quantize_pack_w2(codes, stream=None):
    """int8 codes [N,K] in [-2,1] -> uint8 [N,K/4]."""
    dev = _dev(codes)
    N, K = codes.shape
    Wq = torch.empty((N, K // 4), dtype=torch.uint8, device=dev)
    L.check("quantize_pack_w2", L.load().quantize_pack_w2(_ptr(codes), N, K, _ptr(Wq),
                                                          _stream(stream)))
    return Wq


def ternary_scale_f16(src, stream=None):
    """float32 tensor -> fp16 [1] device tensor holding fp16(mean|src|)."""
    dev = _dev(src)
    out = torch.empty(1, dtype=torch.float16, device=dev)
    L.check("ternary_scale_f16", L.load().ternary_scale_f16(_ptr(src), src.numel(), _ptr(out),
                                                            _stream(stream)))
    return out


def prepack_bytes(layout, N, K):
    return int(L.load().prepack_bytes(layout, N, K))


def prepack_w(layout, Wq, N, K, scales=None, zeros=None, stream=None):
    """Canonical packed codes (+ group scales/zeros) -> opaque prepacked uint8 buffer."""
    dev = _dev(Wq)
    nbytes = prepack_bytes(layout, N, K)
    if nbytes == 0:
        raise L.W4Error("prepack_bytes", L.W4_ERR_SHAPE)
    Wp = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    L.check("prepack_w", L.load().prepack_w(layout, _ptr(Wq), _ptr(scales), _ptr(zeros), N, K,
                                            _ptr(Wp), _stream(stream)))
    return Wp


def unprepack_w(layout, Wp, N, K, stream=None):
    """Inverse of prepack_w -> (Wq, scales-or-None, zeros-or-None)."""
    dev = _dev(Wp)
    rowbytes = {L.W4_LAYOUT_W2A8: K // 4, L.W4_LAYOUT_W8A8: K}.get(layout, K // 2)
    Wq = torch.empty((N, rowbytes), dtype=torch.uint8, device=dev)
    scales = zeros = None
    if layout == L.W4_LAYOUT_W4A16:
        G = K // L.W4_GROUP_SIZE
        scales = torch.empty((N, G), dtype=torch.float16, device=dev)
        zeros = torch.empty((N, G), dtype=torch.uint8, device=dev)
    L.check("unprepack_w", L.load().unprepack_w(layout, _ptr(Wp), N, K, _ptr(Wq), _ptr(scales),
                                                _ptr(zeros), _stream(stream)))
    return Wq, scales, zeros


def quantize_a8(A, with_rowsum=True, out=None, stream=None):
    """fp16/float32 [M,K] -> (Aq int8 [M,K], a_scale float32 [M], rowsum int32 [M] or None)."""
    dev = _dev(A)
    M, K = A.shape
    if A.dtype == torch.float16:
        dt = L.W4_IN_F16
    elif A.dtype == torch.float32:
        dt = L.W4_IN_F32
    else:
        raise ValueError("A must be float16 or float32")
    if out is None:
        Aq = torch.empty((M, K), dtype=torch.int8, device=dev)
        sa = torch.empty(M, dtype=torch.float32, device=dev)
        rs = torch.empty(M, dtype=torch.int32, device=dev) if with_rowsum else None
    else:
        Aq, sa, rs = out
    L.check("quantize_a8", L.load().quantize_a8(_ptr(A), dt, M, K, _ptr(Aq), _ptr(sa), _ptr(rs),
                                                _stream(stream)))
    return Aq, sa, rs


_WS_CACHE = {}


def w4_workspace_bytes(layout, M, N, K):
    key = (layout, M, N, K)
    v = _WS_CACHE.get(key)
    if v is None:
        v = _WS_CACHE[key] = int(L.load().w4_workspace_bytes(layout, M, N, K))
    return v


def w4_plan_workspace_bytes(op, M, N, K):
    """Workspace bytes of a call of ``op`` (W4_OP_*) under the plan in force."""
    key = ("op", op, M, N, K)
    v = _WS_CACHE.get(key)
    if v is None:
        v = _WS_CACHE[key] = int(L.load().w4_plan_workspace_bytes(op, M, N, K))
    return v


_OUT_DT = {L.W4_OUT_F16: torch.float16, L.W4_OUT_F32: torch.float32, L.W4_OUT_I32: torch.int32,
           L.W4_OUT_I8: torch.int8}


def _workspace(ws, op, M, N, K, dev):
    need = w4_plan_workspace_bytes(op, M, N, K)
    if need == 0:
        return None, 0
    if ws is None:
        ws = Workspace(dev)
    buf = ws.get(need) if isinstance(ws, Workspace) else ws
    return buf, buf.numel()


def w4a8_gemm(Aq, a_scale, Wp, w_scale, N, bias=None, out_dtype=L.W4_OUT_F16, workspace=None,
              C=None, stream=None):
    dev = _dev(Aq)
    M, K = Aq.shape
    if C is None:
        C = torch.empty((M, N), dtype=_OUT_DT[out_dtype], device=dev)
    buf, nb = _workspace(workspace, L.W4_OP_W4A8, M, N, K, dev)
    L.check("w4a8_gemm", L.load().w4a8_gemm(_ptr(Aq), _ptr(a_scale), _ptr(Wp), _ptr(w_scale),
                                            _ptr(bias), _ptr(C), out_dtype, M, N, K, _ptr(buf), nb,
                                            _stream(stream)))
    return C


def w2a8_gemm(Aq, a_scale, Wp, w_scale16, N, bias=None, out_dtype=L.W4_OUT_F16, workspace=None,
              C=None, stream=None):
    dev = _dev(Aq)
    M, K = Aq.shape
    if C is None:
        C = torch.empty((M, N), dtype=_OUT_DT[out_dtype], device=dev)
    buf, nb = _workspace(workspace, L.W4_OP_W2A8, M, N, K, dev)
    L.check("w2a8_gemm", L.load().w2a8_gemm(_ptr(Aq), _ptr(a_scale), _ptr(Wp), _ptr(w_scale16),
                                            _ptr(bias), _ptr(C), out_dtype, M, N, K, _ptr(buf), nb,
                                            _stream(stream)))
    return C


def w4a16_gemm(A, Wp, N, bias=None, workspace=None, C=None, group_size=L.W4_GROUP_SIZE,
               stream=None):
    dev = _dev(A)
    M, K = A.shape
    if C is None:
        C = torch.empty((M, N), dtype=torch.float16, device=dev)
    buf, nb = _workspace(workspace, L.W4_OP_W4A16, M, N, K, dev)
    L.check("w4a16_gemm", L.load().w4a16_gemm(_ptr(A), _ptr(Wp), group_size, _ptr(bias), _ptr(C),
                                              M, N, K, _ptr(buf), nb, _stream(stream)))
    return C


def w2a16_gemm(A, Wp, w_scale16, N, bias=None, workspace=None, C=None, stream=None):
    """fp16 A [M,K] x ternary weights (the W2A8 prepacked buffer) -> fp16 C [M,N]."""
    dev = _dev(A)
    M, K = A.shape
    if C is None:
        C = torch.empty((M, N), dtype=torch.float16, device=dev)
    buf, nb = _workspace(workspace, L.W4_OP_W2A16, M, N, K, dev)
    L.check("w2a16_gemm", L.load().w2a16_gemm(_ptr(A), _ptr(Wp), _ptr(w_scale16), _ptr(bias),
                                              _ptr(C), M, N, K, _ptr(buf), nb, _stream(stream)))
    return C

def quantize_pack_w8(W, stream=None):
    """float32 [N,K] -> (Wq int8 [N,K], scales float32 [N]): symmetric INT8 per row."""
    dev = _dev(W)
    N, K = W.shape
    Wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    scales = torch.empty(N, dtype=torch.float32, device=dev)
    L.check("quantize_pack_w8", L.load().quantize_pack_w8(_ptr(W), N, K, _ptr(Wq), _ptr(scales),
                                                          _stream(stream)))
    return Wq, scales


def w8a8_gemm(Aq, a_scale, Wp, w_scale, N, bias=None, out_dtype=L.W4_OUT_F16, out_scale=None,
              workspace=None, C=None, stream=None):
    """INT8 x INT8; out_dtype W4_OUT_I8 re-quantizes by out_scale (device float32 [1])."""
    dev = _dev(Aq)
    M, K = Aq.shape
    if C is None:
        C = torch.empty((M, N), dtype=_OUT_DT[out_dtype], device=dev)
    buf, nb = _workspace(workspace, L.W4_OP_W8A8, M, N, K, dev)
    L.check("w8a8_gemm", L.load().w8a8_gemm(_ptr(Aq), _ptr(a_scale), _ptr(Wp), _ptr(w_scale),
                                            _ptr(bias), _ptr(out_scale), _ptr(C), out_dtype, M, N,
                                            K, _ptr(buf), nb, _stream(stream)))
    return C


def quantize_f8(X, stream=None):
    """fp16/float32 [R,K] -> (codes uint8 [R,K] E4M3, scales float32 [R]), per row."""
    dev = _dev(X)
    R, K = X.shape
    if X.dtype == torch.float16:
        dt = L.W4_IN_F16
    elif X.dtype == torch.float32:
        dt = L.W4_IN_F32
    else:
        raise ValueError("X must be float16 or float32")
    Xq = torch.empty((R, K), dtype=torch.uint8, device=dev)
    scales = torch.empty(R, dtype=torch.float32, device=dev)
    L.check("quantize_f8", L.load().quantize_f8(_ptr(X), dt, R, K, _ptr(Xq), _ptr(scales),
                                                _stream(stream)))
    return Xq, scales


def f8f8_gemm(Aq, a_scale, Wp, w_scale, N, bias=None, out_dtype=L.W4_OUT_F16, workspace=None,
              C=None, stream=None):
    """FP8 E4M3 x FP8 E4M3 (Wp: prepack_w(W4_LAYOUT_W8A8) of E4M3 codes)."""
    dev = _dev(Aq)
    M, K = Aq.shape
    if C is None:
        C = torch.empty((M, N), dtype=_OUT_DT[out_dtype], device=dev)
    buf, nb = _workspace(workspace, L.W4_OP_F8F8, M, N, K, dev)
    L.check("f8f8_gemm", L.load().f8f8_gemm(_ptr(Aq), _ptr(a_scale), _ptr(Wp), _ptr(w_scale),
                                            _ptr(bias), _ptr(C), out_dtype, M, N, K, _ptr(buf),
                                            nb, _stream(stream)))
    return C


_FWS_CACHE = {}


def w4_plan_count(op, M, N, K):
    """Number of candidate plans for (op, M, N, K); op is one of W4_OP_*."""
    n = int(L.load().w4_plan_count(op, M, N, K))
    if n < 0:
        L.check("w4_plan_count", n)
    return n


def w4_plan_name(op, M, N, K, index):
    """Name of candidate ``index`` ("decode:ksplit=S", "skinny", "gemm:RxC")."""
    buf = ctypes.create_string_buffer(64)
    L.check("w4_plan_name", L.load().w4_plan_name(op, M, N, K, index, buf, len(buf)))
    return buf.value.decode()


def _plans_changed():
    # pins change the workspace sizes of their shapes
    _WS_CACHE.clear()
    _FWS_CACHE.clear()


def w4_plan_pin(op, M, N, K, index):
    """Pin candidate ``index`` for the shape (-1 removes the pin)."""
    L.check("w4_plan_pin", L.load().w4_plan_pin(op, M, N, K, index))
    _plans_changed()


def w4_plan_current(op, M, N, K):
    """Index of the candidate a call of this shape runs now."""
    i = int(L.load().w4_plan_current(op, M, N, K))
    if i < 0:
        L.check("w4_plan_current", i)
    return i


def w4_plan_reset():
    """Remove every pinned plan."""
    L.check("w4_plan_reset", L.load().w4_plan_reset())
    _plans_changed()


def w4_fused_act_workspace_bytes(layout, M, N, K):
    key = (layout, M, N, K)
    v = _FWS_CACHE.get(key)
    if v is None:
        v = _FWS_CACHE[key] = int(L.load().w4_fused_act_workspace_bytes(layout, M, N, K))
    return v


def _fused(name, layout, A, Wp, scale, N, bias, out_dtype, workspace, C, stream):
    dev = _dev(A)
    M, K = A.shape
    if A.dtype == torch.float16:
        dt = L.W4_IN_F16
    elif A.dtype == torch.float32:
        dt = L.W4_IN_F32
    else:
        raise ValueError("A must be float16 or float32")
    if C is None:
        C = torch.empty((M, N), dtype=_OUT_DT[out_dtype], device=dev)
    need = w4_fused_act_workspace_bytes(layout, M, N, K)
    buf, nb = None, 0
    if need:
        if workspace is None:
            workspace = Workspace(dev)
        buf = workspace.get(need) if isinstance(workspace, Workspace) else workspace
        nb = buf.numel()
    L.check(name, getattr(L.load(), name)(_ptr(A), dt, _ptr(Wp), _ptr(scale), _ptr(bias), _ptr(C),
                                          out_dtype, M, N, K, _ptr(buf), nb, _stream(stream)))
    return C


def w4a8_gemm_fused_act(A, Wp, w_scale, N, bias=None, out_dtype=L.W4_OUT_F16, workspace=None,
                        C=None, stream=None):
    """fp16/float32 A [M,K] -> quantize_a8 + w4a8_gemm in one C call."""
    return _fused("w4a8_gemm_fused_act", L.W4_LAYOUT_W4A8, A, Wp, w_scale, N, bias, out_dtype,
                  workspace, C, stream)


def w2a8_gemm_fused_act(A, Wp, w_scale16, N, bias=None, out_dtype=L.W4_OUT_F16, workspace=None,
                        C=None, stream=None):
    """fp16/float32 A [M,K] -> quantize_a8 + w2a8_gemm in one C call."""
    return _fused("w2a8_gemm_fused_act", L.W4_LAYOUT_W2A8, A, Wp, w_scale16, N, bias, out_dtype,
                  workspace, C, stream)
