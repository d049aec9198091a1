"""torch-tensor wrappers with the C entry points' names (marshalling only)."""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L


def _ptr(t):
    return None if t is None else t.data_ptr()


def _tstream(stream):
    """The torch stream a call runs on (None: the current stream)."""
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream):
    return _tstream(stream).cuda_stream


def _empty(shape, dtype, dev, stream):
    """An output buffer from the caching pool of the stream the kernel runs on,
    so that the pool hands the memory out again only behind that kernel."""
    with torch.cuda.stream(_tstream(stream)):
        return torch.empty(shape, dtype=dtype, device=dev)


def _dev(t):
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.device


class Workspace:
    """A zero-filled device workspace that grows on demand.

    The matmul kernels leave the part they rely on zero after each call, so
    one workspace serves any number of calls issued on one stream. The buffer
    is allocated and zero-filled on the stream of the call that needs it; a
    call on another stream first waits for the stream that used it last, so
    calls sharing a workspace never overlap.
    """

    def __init__(self, device=None):
        self.device = torch.device(device or "cuda")
        self.buf = None
        self.stream = None          # the stream that used the buffer last
        self.alloc_stream = None    # the stream the buffer was allocated on

    def get(self, nbytes, stream=None):
        if nbytes == 0:
            return None
        s = _tstream(stream)
        if self.buf is None or self.buf.numel() < nbytes:
            if self.buf is not None and self.stream is not None and self.stream != s:
                s.wait_stream(self.stream)      # the old buffer's last user first
            with torch.cuda.stream(s):
                self.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            self.alloc_stream = s
        elif self.stream is not None and self.stream != s:
            s.wait_stream(self.stream)
        if s != self.alloc_stream:
            # keep the pool from handing the memory out while s may still use it
            self.buf.record_stream(s)
        self.stream = s
        return self.buf


def quantize_pack_w4(W, scheme=L.W4_SYM_PER_CHANNEL, group_size=None, stream=None):
    """float32 [N,K] -> (Wq uint8 [N,K/2], scales, zeros-or-None)."""
    dev = _dev(W)
    N, K = W.shape
    Wq = _empty((N, K // 2), torch.uint8, dev, stream)
    if scheme == L.W4_SYM_PER_CHANNEL:
        gs = -1 if group_size is None else group_size
        scales = _empty(N, torch.float32, dev, stream)
        zeros = None
    else:
        gs = L.W4_GROUP_SIZE if group_size is None else group_size
        G = K // L.W4_GROUP_SIZE
        scales = _empty((N, G), torch.float16, dev, stream)
        zeros = _empty((N, G), torch.uint8, dev, stream)
    L.check("quantize_pack_w4", L.load().quantize_pack_w4(
        _ptr(W), N, K, scheme, gs, _ptr(Wq), _ptr(scales), _ptr(zeros), _stream(stream)))
    return Wq, scales, zeros


def quantize_pack_w2(codes, stream=None):
    """int8 codes [N,K] in [-2,1] -> uint8 [N,K/4]."""
    dev = _dev(codes)
    N, K = codes.shape
    Wq = _empty((N, K // 4), torch.uint8, dev, stream)
    L.check("quantize_pack_w2", L.load().quantize_pack_w2(_ptr(codes), N, K, _ptr(Wq),
                                                          _stream(stream)))
    return Wq


def ternary_scale_f16(src, stream=None):
    """float32 tensor -> fp16 [1] device tensor holding fp16(mean|src|)."""
    dev = _dev(src)
    out = _empty(1, torch.float16, dev, stream)
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
    Wp = _empty(nbytes, torch.uint8, dev, stream)
    L.check("prepack_w", L.load().prepack_w(layout, _ptr(Wq), _ptr(scales), _ptr(zeros), N, K,
                                            _ptr(Wp), _stream(stream)))
    return Wp


def unprepack_w(layout, Wp, N, K, stream=None):
    """Inverse of prepack_w -> (Wq, scales-or-None, zeros-or-None)."""
    dev = _dev(Wp)
    rowbytes = {L.W4_LAYOUT_W2A8: K // 4, L.W4_LAYOUT_W8A8: K}.get(layout, K // 2)
    Wq = _empty((N, rowbytes), torch.uint8, dev, stream)
    scales = zeros = None
    if layout == L.W4_LAYOUT_W4A16:
        G = K // L.W4_GROUP_SIZE
        scales = _empty((N, G), torch.float16, dev, stream)
        zeros = _empty((N, G), torch.uint8, dev, stream)
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
        Aq = _empty((M, K), torch.int8, dev, stream)
        sa = _empty(M, torch.float32, dev, stream)
        rs = _empty(M, torch.int32, dev, stream) if with_rowsum else None
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


def _workspace(ws, op, M, N, K, dev, stream):
    need = w4_plan_workspace_bytes(op, M, N, K)
    if need == 0:
        return None, 0
    if ws is None:
        ws = Workspace(dev)
    buf = ws.get(need, stream) if isinstance(ws, Workspace) else ws
    return buf, buf.numel()


def w4a8_gemm(Aq, a_scale, Wp, w_scale, N, bias=None, out_dtype=L.W4_OUT_F16, workspace=None,
              C=None, stream=None):
    dev = _dev(Aq)
    M, K = Aq.shape
    if C is None:
        C = _empty((M, N), _OUT_DT[out_dtype], dev, stream)
    buf, nb = _workspace(workspace, L.W4_OP_W4A8, M, N, K, dev, stream)
    L.check("w4a8_gemm", L.load().w4a8_gemm(_ptr(Aq), _ptr(a_scale), _ptr(Wp), _ptr(w_scale),
                                            _ptr(bias), _ptr(C), out_dtype, M, N, K, _ptr(buf), nb,
                                            _stream(stream)))
    return C


def w2a8_gemm(Aq, a_scale, Wp, w_scale16, N, bias=None, out_dtype=L.W4_OUT_F16, workspace=None,
              C=None, stream=None):
    dev = _dev(Aq)
    M, K = Aq.shape
    if C is None:
        C = _empty((M, N), _OUT_DT[out_dtype], dev, stream)
    buf, nb = _workspace(workspace, L.W4_OP_W2A8, M, N, K, dev, stream)
    L.check("w2a8_gemm", L.load().w2a8_gemm(_ptr(Aq), _ptr(a_scale), _ptr(Wp), _ptr(w_scale16),
                                            _ptr(bias), _ptr(C), out_dtype, M, N, K, _ptr(buf), nb,
                                            _stream(stream)))
    return C


def w4a16_gemm(A, Wp, N, bias=None, workspace=None, C=None, group_size=L.W4_GROUP_SIZE,
               stream=None):
    dev = _dev(A)
    M, K = A.shape
    if C is None:
        C = _empty((M, N), torch.float16, dev, stream)
    buf, nb = _workspace(workspace, L.W4_OP_W4A16, M, N, K, dev, stream)
    L.check("w4a16_gemm", L.load().w4a16_gemm(_ptr(A), _ptr(Wp), group_size, _ptr(bias), _ptr(C),
                                              M, N, K, _ptr(buf), nb, _stream(stream)))
    return C


def w2a16_gemm(A, Wp, w_scale16, N, bias=None, workspace=None, C=None, stream=None):
    """fp16 A [M,K] x ternary weights (the W2A8 prepacked buffer) -> fp16 C [M,N]."""
    dev = _dev(A)
    M, K = A.shape
    if C is None:
        C = _empty((M, N), torch.float16, dev, stream)
    buf, nb = _workspace(workspace, L.W4_OP_W2A16, M, N, K, dev, stream)
    L.check("w2a16_gemm", L.load().w2a16_gemm(_ptr(A), _ptr(Wp), _ptr(w_scale16), _ptr(bias),
                                              _ptr(C), M, N, K, _ptr(buf), nb, _stream(stream)))
    return C

def quantize_pack_w8(W, stream=None):
    """float32 [N,K] -> (Wq int8 [N,K], scales float32 [N]): symmetric INT8 per row."""
    dev = _dev(W)
    N, K = W.shape
    Wq = _empty((N, K), torch.int8, dev, stream)
    scales = _empty(N, torch.float32, dev, stream)
    L.check("quantize_pack_w8", L.load().quantize_pack_w8(_ptr(W), N, K, _ptr(Wq), _ptr(scales),
                                                          _stream(stream)))
    return Wq, scales


def w8a8_gemm(Aq, a_scale, Wp, w_scale, N, bias=None, out_dtype=L.W4_OUT_F16, out_scale=None,
              workspace=None, C=None, stream=None):
    """INT8 x INT8; out_dtype W4_OUT_I8 re-quantizes by out_scale (device float32 [1])."""
    dev = _dev(Aq)
    M, K = Aq.shape
    if C is None:
        C = _empty((M, N), _OUT_DT[out_dtype], dev, stream)
    buf, nb = _workspace(workspace, L.W4_OP_W8A8, M, N, K, dev, stream)
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
    Xq = _empty((R, K), torch.uint8, dev, stream)
    scales = _empty(R, torch.float32, dev, stream)
    L.check("quantize_f8", L.load().quantize_f8(_ptr(X), dt, R, K, _ptr(Xq), _ptr(scales),
                                                _stream(stream)))
    return Xq, scales


def f8f8_gemm(Aq, a_scale, Wp, w_scale, N, bias=None, out_dtype=L.W4_OUT_F16, workspace=None,
              C=None, stream=None):
    """FP8 E4M3 x FP8 E4M3 (Wp: prepack_w(W4_LAYOUT_W8A8) of E4M3 codes)."""
    dev = _dev(Aq)
    M, K = Aq.shape
    if C is None:
        C = _empty((M, N), _OUT_DT[out_dtype], dev, stream)
    buf, nb = _workspace(workspace, L.W4_OP_F8F8, M, N, K, dev, stream)
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
        C = _empty((M, N), _OUT_DT[out_dtype], dev, stream)
    need = w4_fused_act_workspace_bytes(layout, M, N, K)
    buf, nb = None, 0
    if need:
        if workspace is None:
            workspace = Workspace(dev)
        buf = workspace.get(need, stream) if isinstance(workspace, Workspace) else workspace
        nb = buf.numel()
    L.check(name, getattr(L.load(), name)(_ptr(A), dt, _ptr(Wp), _ptr(scale), _ptr(bias), _ptr(C),
                                          out_dtype, M, N, K, _ptr(buf), nb, _stream(stream)))
    return C


def w4a8_gemm_fused_act(A, Wp, w_scale, N, bias=None, out_dtype=L.W4_OUT_F16, workspace=None,
                        C=None, stream=None):
    """fp16/float32 A [M,K] -> quantize_a8 + w4a8_gemm in one C call."""
    return _fused("w4a8_gemm_fused_act", L.W4_LAYOUT_W4A8, A, Wp, w_scale, N, bias, out_dtype,
                  workspace, C, stream)


def w4a8_gemm_fused_act_noalloc(A, Wp, w_scale, N, bias=None, out_dtype=L.W4_OUT_F16, C=None,
                                stream=None):
    """w4a8_gemm_fused_act on the library's static per-GPU scratch: no
    workspace is allocated (pass ``C`` as well to allocate nothing at all)."""
    dev = _dev(A)
    M, K = A.shape
    if A.dtype == torch.float16:
        dt = L.W4_IN_F16
    elif A.dtype == torch.float32:
        dt = L.W4_IN_F32
    else:
        raise ValueError("A must be float16 or float32")
    if C is None:
        C = _empty((M, N), _OUT_DT[out_dtype], dev, stream)
    L.check("w4a8_gemm_fused_act_noalloc", L.load().w4a8_gemm_fused_act_noalloc(
        _ptr(A), dt, _ptr(Wp), _ptr(w_scale), _ptr(bias), _ptr(C), out_dtype, M, N, K,
        _stream(stream)))
    return C


def w2a8_gemm_fused_act(A, Wp, w_scale16, N, bias=None, out_dtype=L.W4_OUT_F16, workspace=None,
                        C=None, stream=None):
    """fp16/float32 A [M,K] -> quantize_a8 + w2a8_gemm in one C call."""
    return _fused("w2a8_gemm_fused_act", L.W4_LAYOUT_W2A8, A, Wp, w_scale16, N, bias, out_dtype,
                  workspace, C, stream)


def w4_read_probe(buf, nbytes=None, per=4, sink=None, stream=None):
    """Read ``nbytes`` (default: all) of the uint8 device tensor ``buf`` once
    with 16-byte loads: the plain streaming read a weight-streaming kernel of
    the same size is measured against. ``sink`` is a device uint32 [1024]."""
    dev = _dev(buf)
    nbytes = buf.numel() * buf.element_size() if nbytes is None else nbytes
    if sink is None:
        sink = _empty(1024, torch.int32, dev, stream)
    L.check("w4_read_probe", L.load().w4_read_probe(_ptr(buf), nbytes, per, _ptr(sink),
                                                    _stream(stream)))
    return sink


class StepGraph:
    """A decode step captured once and launched as one HIP graph, its kernels
    re-pointed at each step's buffers by a kernel-node parameter update (the
    C calls w4_graph_*; INT4 quantization page, Part 2, steps 2-4)::

        g = StepGraph(stream)            # a torch.cuda.Stream of the caller
        with g.capture():                # the library calls of one step
            step(buffers_0)
        g.launch()
        with g.update():                 # the same calls, the next buffers
            step(buffers_1)
        g.launch()

    Inside ``capture`` and ``update`` the calls run on ``stream`` (it is made
    the current stream) and are recorded, not run. Outputs and workspaces must
    be allocated beforehand: nothing may be allocated while capturing.
    """

    def __init__(self, stream):
        if stream is None or stream.cuda_stream == 0:
            raise ValueError("StepGraph needs a stream created by the caller")
        self.stream = stream
        self.handle = None

    def _capture(self, name, finish):
        lib = L.load()
        parent = self

        class _Ctx:
            def __enter__(self):
                self.ctx = torch.cuda.stream(parent.stream)
                self.ctx.__enter__()
                try:
                    L.check("w4_graph_begin", lib.w4_graph_begin(parent.stream.cuda_stream))
                except BaseException:
                    self.ctx.__exit__(None, None, None)
                    raise
                return parent

            def __exit__(self, et, ev, tb):
                try:
                    if et is None:
                        status = finish(lib)
                    else:
                        # the step raised: end the capture and discard it
                        h = ctypes.c_void_p()
                        if lib.w4_graph_end(parent.stream.cuda_stream, ctypes.byref(h)) == L.W4_OK:
                            lib.w4_graph_destroy(h.value)
                finally:
                    self.ctx.__exit__(et, ev, tb)
                if et is None:
                    L.check(name, status)
                return False
        return _Ctx()

    def capture(self):
        """Context: capture one step and instantiate it."""
        if self.handle is not None:
            raise RuntimeError("already captured; use update()")

        def finish(lib):
            h = ctypes.c_void_p()
            st = lib.w4_graph_end(self.stream.cuda_stream, ctypes.byref(h))
            if st == L.W4_OK:
                self.handle = h.value
            return st
        return self._capture("w4_graph_end", finish)

    def update(self):
        """Context: capture the same step with other buffers and update the
        instantiated graph's kernel nodes from it (W4Error W4_ERR_ARG if the
        calls differ in kernels, grids or shapes; the graph is then unchanged)."""
        if self.handle is None:
            raise RuntimeError("nothing captured yet")
        return self._capture(
            "w4_graph_update",
            lambda lib: lib.w4_graph_update(self.handle, self.stream.cuda_stream))

    def launch(self, stream=None):
        """Launch the graph on ``stream`` (default: the capture stream)."""
        s = self.stream if stream is None else stream
        L.check("w4_graph_launch", L.load().w4_graph_launch(self.handle, s.cuda_stream))

    def kernel_nodes(self):
        n = L.load().w4_graph_kernel_nodes(self.handle)
        if n < 0:
            L.check("w4_graph_kernel_nodes", n)
        return n

    def close(self):
        if self.handle is not None:
            L.check("w4_graph_destroy", L.load().w4_graph_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
