"""GPU: decode-step graphs built by the library (w4_graph_*), after the INT4
quantization page, Part 2 (capture, instantiate, update the kernel-node
parameters so the captured step reads and writes the current step's buffers,
launch the graph). Every launch is checked against the oracle."""
import numpy as np
import pytest

import oracle as O
from gemv_nibble_unpack_amd import workloads as WL
from tests._helpers import say, tol_ok
from tests.test_gpu_parity import dev, g, host, prep_w2a8, prep_w4a8, prep_w4a16  # noqa: F401

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _chain(g, dims, kinds, seed):
    """Layers of a decode step (fp16 output of one feeds the next) and the
    oracle of each layer."""
    layers, refs = [], []
    for i, kind in enumerate(kinds):
        K, N = dims[i], dims[i + 1]
        W = WL.weights_f32(N, K, seed=seed + i)
        if kind == "w4a16":
            layers.append((kind, prep_w4a16(g, W), None, N))
            q, s16, z = O.quantize_w4_group(W, 128)
            refs.append(lambda x, q=q, s16=s16, z=z: O.w4a16_gemm(x, q, s16, z, 128))
        elif kind == "w4a8":
            Wp, ws = prep_w4a8(g, W)
            layers.append((kind, Wp, ws, N))
            qw, sw = O.quantize_w4_sym(W)

            def ref_w4a8(x, qw=qw, sw=sw):
                qa, sa, _ = O.quantize_a8(x)
                return O.w4a8_gemm(qa, sa, qw, sw, None, O.OUT_F16)
            refs.append(ref_w4a8)
        else:
            codes = WL.ternary_codes(N, K, seed=seed + 100 + i)
            Wp, ws = prep_w2a8(g, codes, W)
            layers.append((kind, Wp, ws, N))

            def ref_w2a8(x, codes=codes, ws=ws):
                qa, sa, _ = O.quantize_a8(x)
                return O.w2a8_gemm(qa, sa, codes, host(ws)[0], None, O.OUT_F16)
            refs.append(ref_w2a8)
    return layers, refs


def _run(g, layers, bufs, wss):
    for i, (kind, Wp, ws, N) in enumerate(layers):
        if kind == "w4a16":
            g.w4a16_gemm(bufs[i], Wp, N, workspace=wss[i], C=bufs[i + 1])
        elif kind == "w4a8":
            g.w4a8_gemm_fused_act(bufs[i], Wp, ws, N, workspace=wss[i], C=bufs[i + 1])
        else:
            g.w2a8_gemm_fused_act(bufs[i], Wp, ws, N, workspace=wss[i], C=bufs[i + 1])


def _check(bufs, refs, what):
    outs = [host(b) for b in bufs[1:]]
    ins = [host(bufs[0])] + outs[:-1]
    for i, ref in enumerate(refs):
        assert np.isfinite(outs[i].astype(np.float32)).all(), (what, i)
        tol_ok(outs[i], ref(ins[i]), f"{what}: layer {i}")
    return outs


def test_step_graph_repoints_a_decode_chain(g):
    # One step of a decode chain (W4A16, fused W4A8, W4A16 with a k split,
    # fused W2A8) captured once; the graph is then re-pointed, by kernel-node
    # parameter updates, at two other sets of input/output buffers and back,
    # and every launch is checked against the oracle, as are the buffers a
    # launch must not touch.
    say("case step graph: decode chain with node-parameter updates")
    dims = [4096, 11008, 4096, 256, 3200]
    kinds = ["w4a16", "w4a8", "w4a16", "w2a8"]
    layers, refs = _chain(g, dims, kinds, seed=9400)
    sets = [[torch.empty((1, d), dtype=torch.float16, device="cuda") for d in dims]
            for _ in range(3)]
    xs = [dev(WL.activations(1, dims[0], seed=9500 + j, dtype=np.float16)) for j in range(3)]
    for bufs, x in zip(sets, xs):
        bufs[0].copy_(x)
    wss = [g.Workspace("cuda") for _ in layers]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _run(g, layers, sets[0], wss)                # sizes the workspaces before capture
    s.synchronize()
    for b in sets[0][1:]:
        b.fill_(0)
    torch.cuda.synchronize()

    graph = g.StepGraph(s)
    with graph.capture():
        _run(g, layers, sets[0], wss)
    # one or two kernels per call (a fused call may quantize in a kernel of its own)
    assert graph.kernel_nodes() >= len(layers)
    torch.cuda.synchronize()
    for b in sets[0][1:]:
        assert not host(b).any()                     # captured, not run
    graph.launch()
    s.synchronize()
    first = _check(sets[0], refs, "launch 0")

    for j in (1, 2, 0):
        for b in sets[j][1:]:
            b.fill_(0)
        before = [[host(b).copy() for b in sets[k][1:]] for k in range(3) if k != j]
        torch.cuda.synchronize()
        with graph.update():
            _run(g, layers, sets[j], wss)
        graph.launch()
        s.synchronize()
        outs = _check(sets[j], refs, f"launch re-pointed at set {j}")
        if j == 0:                                   # back to the first buffers
            for o, f in zip(outs, first):
                assert np.array_equal(o.view(np.uint16), f.view(np.uint16))
        after = [[host(b) for b in sets[k][1:]] for k in range(3) if k != j]
        for bb, aa in zip(before, after):            # the other sets untouched
            for x, y in zip(bb, aa):
                assert np.array_equal(x.view(np.uint16), y.view(np.uint16))
    graph.close()


def test_step_graph_refuses_an_update_from_another_step(g):
    # A capture of other kernels (another shape, so other grids) cannot update
    # the graph: W4_ERR_ARG, and the graph still computes its own step.
    say("case step graph: mismatched update refused")
    dims = [1024, 2048, 512]
    layers, refs = _chain(g, dims, ["w4a16", "w4a8"], seed=9600)
    other, _ = _chain(g, [1024, 4096, 512], ["w4a16", "w4a8"], seed=9700)
    bufs = [torch.empty((1, d), dtype=torch.float16, device="cuda") for d in dims]
    obufs = [torch.empty((1, d), dtype=torch.float16, device="cuda") for d in (1024, 4096, 512)]
    bufs[0].copy_(dev(WL.activations(1, dims[0], seed=9800, dtype=np.float16)))
    obufs[0].copy_(bufs[0])
    wss = [g.Workspace("cuda") for _ in layers]
    owss = [g.Workspace("cuda") for _ in other]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _run(g, layers, bufs, wss)
        _run(g, other, obufs, owss)
    s.synchronize()
    graph = g.StepGraph(s)
    with graph.capture():
        _run(g, layers, bufs, wss)
    with pytest.raises(g.W4Error) as e:
        with graph.update():
            _run(g, other, obufs, owss)
    assert e.value.status == -4                       # W4_ERR_ARG
    for b in bufs[1:]:
        b.fill_(0)
    torch.cuda.synchronize()
    graph.launch()
    s.synchronize()
    _check(bufs, refs, "launch after a refused update")
    graph.close()
