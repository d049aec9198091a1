"""GPU parity of the plan table: every candidate plan of a shape against the
oracle, one workspace shared by any mix of shapes and plans, and the tuner.

Every output element is checked. INT32 accumulators and INT8 outputs must
be bit-exact for every plan (the products are exact integers whatever the k
split); fp16 outputs meet the same tolerance as the other parity tests,
|gpu - ref| <= 2^-9 |ref| + 1e-3 rms(ref).
"""
import json

import numpy as np
import pytest

import oracle as O
from gemv_nibble_unpack_amd import workloads as WL
from tests._helpers import say, tol_ok

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemv_nibble_unpack_amd as G
    G.load()
    G.w4_plan_reset()
    yield G
    G.w4_plan_reset()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def f16(x):
    return dev(np.asarray(x, np.float16))


class Shape:
    """Operands of one (op, M, N, K) on the device plus the oracle's view."""

    def __init__(self, g, op, M, N, K, seed):
        self.g, self.op, self.M, self.N, self.K = g, op, M, N, K
        self.A = WL.activations(M, K, seed=seed, dtype=np.float16)
        self.bias = WL.bias_f16(N, seed=seed + 1)
        a8 = op in (g.W4_OP_W4A8, g.W4_OP_W2A8, g.W4_OP_W8A8)
        if a8:
            self.Aq, self.sa, _ = g.quantize_a8(dev(self.A))
            self.qa, self.sa_ref, _ = O.quantize_a8(self.A)
        if op == g.W4_OP_F8F8:
            self.Aq, self.sa = g.quantize_f8(dev(self.A))
            self.qa, self.sa_ref = O.quantize_f8(self.A)
            W = WL.weights_f32(N, K, seed=seed + 3)
            Wq, self.scale = g.quantize_f8(dev(W))
            self.Wp = g.prepack_w(g.W4_LAYOUT_W8A8, Wq, N, K)
            self.qw, self.sw = O.quantize_f8(W)
        elif op in (g.W4_OP_W2A8, g.W4_OP_W2A16):
            self.codes = WL.ternary_codes(N, K, seed=seed + 3)
            Wq = g.quantize_pack_w2(dev(self.codes))
            self.Wp = g.prepack_w(g.W4_LAYOUT_W2A8, Wq, N, K)
            self.scale = g.ternary_scale_f16(dev(WL.weights_f32(N, K, seed=seed + 4)))
            s = np.float64(host(self.scale)[0])
            self.qw, self.ws_ref = self.codes, np.full((1, N), s)
        elif op == g.W4_OP_W4A16:
            W = WL.weights_f32(N, K, seed=seed + 3)
            Wq, s, z = g.quantize_pack_w4(dev(W), g.W4_ASYM_GROUP)
            self.Wp = g.prepack_w(g.W4_LAYOUT_W4A16, Wq, N, K, s, z)
            self.q, self.s16, self.z = O.quantize_w4_group(W, 128)
        elif op == g.W4_OP_W8A8:
            W = WL.weights_f32(N, K, seed=seed + 3)
            Wq, self.scale = g.quantize_pack_w8(dev(W))
            self.Wp = g.prepack_w(g.W4_LAYOUT_W8A8, Wq, N, K)
            self.qw, ws = O.quantize_w8_sym(W)
            self.ws_ref = ws[None, :]
        else:
            W = WL.weights_f32(N, K, seed=seed + 3)
            Wq, self.scale, _ = g.quantize_pack_w4(dev(W), g.W4_SYM_PER_CHANNEL)
            self.Wp = g.prepack_w(g.W4_LAYOUT_W4A8, Wq, N, K)
            self.qw, ws = O.quantize_w4_sym(W)
            self.ws_ref = ws[None, :]
        if a8:
            self.acc = O.int_accumulate_f64(self.qa, self.qw)

    def run(self, out_dtype, bias=False, workspace=None, out_scale=None):
        g, N = self.g, self.N
        b = f16(self.bias) if bias else None
        if self.op == g.W4_OP_W4A16:
            return host(g.w4a16_gemm(dev(self.A), self.Wp, N, bias=b, workspace=workspace))
        if self.op == g.W4_OP_W2A16:
            return host(g.w2a16_gemm(dev(self.A), self.Wp, self.scale, N, bias=b,
                                     workspace=workspace))
        if self.op == g.W4_OP_F8F8:
            return host(g.f8f8_gemm(self.Aq, self.sa, self.Wp, self.scale, N, bias=b,
                                    out_dtype=out_dtype, workspace=workspace))
        mm = {g.W4_OP_W4A8: g.w4a8_gemm, g.W4_OP_W2A8: g.w2a8_gemm}.get(self.op)
        if mm is None:
            return host(g.w8a8_gemm(self.Aq, self.sa, self.Wp, self.scale, N, bias=b,
                                    out_dtype=out_dtype, out_scale=out_scale, workspace=workspace))
        return host(mm(self.Aq, self.sa, self.Wp, self.scale, N, bias=b, out_dtype=out_dtype,
                       workspace=workspace))

    def ref_f16(self, bias=True):
        """The oracle's fp16 output of the whole [M, N] product."""
        b = self.bias if bias else None
        if self.op == self.g.W4_OP_W4A16:
            return O.w4a16_gemm(self.A, self.q, self.s16, self.z, 128, b)
        if self.op == self.g.W4_OP_W2A16:
            return O.w2a16_gemm(self.A, self.codes, np.float64(host(self.scale)[0]), b)
        if self.op == self.g.W4_OP_F8F8:
            return O.f8f8_gemm(self.qa, self.sa_ref, self.qw, self.sw, b, O.OUT_F16)
        return O.dequant_epilogue(self.acc, self.ws_ref, self.sa_ref[:, None],
                                  None if b is None else b[None, :], O.OUT_F16)

    def check(self, what):
        """Every output type of the op against the oracle, every element."""
        g = self.g
        tol_ok(self.run(g.W4_OUT_F16, bias=True), self.ref_f16(), what)
        if self.op == g.W4_OP_F8F8:
            ref = O.f8f8_gemm(self.qa, self.sa_ref, self.qw, self.sw, None, O.OUT_F32)
            tol_ok(self.run(g.W4_OUT_F32), ref, f"{what} f32")
        if self.op in (g.W4_OP_W4A16, g.W4_OP_W2A16, g.W4_OP_F8F8):
            return
        C32 = self.run(g.W4_OUT_I32)
        assert np.array_equal(C32, self.acc.astype(np.int32)), what
        if self.op == g.W4_OP_W8A8:
            vmax = float(np.max(np.abs((self.acc.astype(np.float32) * self.ws_ref) *
                                       self.sa_ref[:, None])))
            so = np.float32(vmax / 100.0)
            C8 = self.run(g.W4_OUT_I8, out_scale=dev(np.array([so], np.float32)))
            assert np.array_equal(C8, O.requantize_i8(self.acc, self.ws_ref,
                                                      self.sa_ref[:, None], so)), what


PLAN_SHAPES = [
    ("w4a8", 1, 4096, 4096), ("w4a8", 37, 1000, 1040), ("w4a8", 130, 4100, 528),
    ("w2a8", 1, 16, 131056), ("w2a8", 70, 3000, 2000),
    # long rows: 16-wave decode plans next to the 8-wave ones (the first two
    # take 16 waves unsplit as their built-in plan; ragged last n-tile)
    ("w4a16", 1, 1040, 11008), ("w2a16", 1, 1030, 8640), ("w8a8", 3, 300, 8192),
    # rows too long to stage: 16-wave plans stream their fragments from L2
    ("w4a16", 13, 1000, 4096), ("w8a8", 9, 700, 4096),
    # one INT8 row over 65 n-tiles: 4-wave plans built in (k tail in the second)
    ("w2a8", 1, 1030, 3200), ("w8a8", 1, 1030, 1008),
    # split GEMM finishes over column pairs with a ragged pair (N % 4 == 2)
    # and over single columns (odd N), with rows past M in the last block
    ("w2a8", 130, 1002, 1024), ("w2a8", 100, 1001, 768),
    ("w4a16", 16, 4096, 4096), ("w4a16", 33, 1000, 1024), ("w4a16", 130, 1003, 512),
    ("w2a16", 3, 3200, 8640), ("w2a16", 40, 3000, 2000),
    ("w8a8", 16, 4096, 4096), ("w8a8", 20, 1000, 528),
    ("f8f8", 16, 4096, 4096), ("f8f8", 20, 1000, 528),
    # the FP8 GEMM candidate with ragged rows, columns and an odd count of
    # 64-k weight tiles with a k tail
    ("f8f8", 130, 1003, 1040),
]


@pytest.mark.parametrize("name,M,N,K", PLAN_SHAPES)
def test_every_plan_matches_oracle(g, name, M, N, K):
    # every candidate: decode at each k split, skinny, and (INT8 activations,
    # M > 16) every GEMM block shape, with ragged M, N and k tails
    op = getattr(g, "W4_OP_" + name.upper())
    s = Shape(g, op, M, N, K, seed=12000 + M + N)
    n = g.w4_plan_count(op, M, N, K)
    assert n >= 2
    exact = op in (g.W4_OP_W4A8, g.W4_OP_W2A8, g.W4_OP_W8A8)
    first = None
    try:
        for i in range(n):
            plan = g.w4_plan_name(op, M, N, K, i)
            say(f"case plan {name} M={M} N={N} K={K} {plan}")
            g.w4_plan_pin(op, M, N, K, i)
            assert g.w4_plan_current(op, M, N, K) == i
            s.check(f"{name} {M}x{N}x{K} {plan}")
            if exact:
                # integer sums do not depend on how K is split: every plan
                # gives the whole INT32 output bit for bit
                full = s.run(g.W4_OUT_I32)
                if first is None:
                    first = full
                else:
                    assert np.array_equal(full, first), plan
    finally:
        g.w4_plan_pin(op, M, N, K, -1)


def test_one_workspace_for_any_mix_of_shapes_and_plans(g):
    # A decode call split 64 ways leaves partial sums past the counter area; a
    # split GEMM (144 output tiles) and a 4-way split decode (256 output
    # tiles) then count arrivals in the same buffer. Each must equal its
    # result on a fresh workspace, bit for bit.
    say("case shared workspace: decode split 64, gemm split, decode split 4")
    cases = [Shape(g, g.W4_OP_W2A8, 1, 16, 131056, seed=13000),
             Shape(g, g.W4_OP_W2A8, 1100, 2000, 1024, seed=13100),
             Shape(g, g.W4_OP_W4A8, 1, 4096, 4096, seed=13200)]
    names = [g.w4_plan_name(c.op, c.M, c.N, c.K, g.w4_plan_current(c.op, c.M, c.N, c.K))
             for c in cases[:2]]
    assert names == ["decode:ksplit=64", "gemm:128x128,ksplit=2"]
    try:
        split4 = [g.w4_plan_name(g.W4_OP_W4A8, 1, 4096, 4096, i)
                  for i in range(g.w4_plan_count(g.W4_OP_W4A8, 1, 4096, 4096))].index(
                      "decode:ksplit=4")
        g.w4_plan_pin(g.W4_OP_W4A8, 1, 4096, 4096, split4)
        need = max(g.w4_plan_workspace_bytes(c.op, c.M, c.N, c.K) for c in cases)
        assert need > 16384
        shared = torch.zeros(need, dtype=torch.uint8, device="cuda")
        for rep in range(2):
            for c in cases:
                got = c.run(g.W4_OUT_I32, workspace=shared)
                fresh = c.run(g.W4_OUT_I32)
                assert np.array_equal(got, fresh), (rep, c.op, c.M, c.N, c.K)
                assert np.array_equal(got, c.acc.astype(np.int32))
        # the counter area is zero again after the calls
        assert not host(shared[:16384]).any()
    finally:
        g.w4_plan_pin(g.W4_OP_W4A8, 1, 4096, 4096, -1)


def test_tuner_pins_a_candidate_and_results_hold(g, tmp_path):
    from gemv_nibble_unpack_amd import tune
    op, M, N, K = g.W4_OP_W4A8, 130, 4100, 528
    say(f"case tune w4a8 M={M} N={N} K={K}")
    try:
        rec = tune.tune_shape(op, M, N, K, reps=5, warmup=1)
        names = tune.candidates(op, M, N, K)
        assert set(rec["candidates"]) == set(names)
        assert rec["plan"] in names and rec["us"] == min(rec["candidates"].values())
        assert names[g.w4_plan_current(op, M, N, K)] == rec["plan"]
        Shape(g, op, M, N, K, seed=14000).check(f"tuned {rec['plan']}")
        # the saved table pins the same plan by name in a clean table
        path = tmp_path / "plans.json"
        tune.save(str(path), [rec])
        assert json.loads(path.read_text())["plans"][0]["plan"] == rec["plan"]
        g.w4_plan_reset()
        assert tune.load(str(path)) == []
        assert names[g.w4_plan_current(op, M, N, K)] == rec["plan"]
    finally:
        g.w4_plan_reset()


@pytest.mark.parametrize("name,M,N,K,plan", [
    ("w4a16", 16, 1024, 4096, "skinny:ksplit=4"),
    ("w2a16", 40, 1000, 2048, "skinny:rows=32,ksplit=4"),
    ("w4a16", 1, 512, 8192, "decode:ksplit=4"),
])
def test_float_split_sums_do_not_depend_on_arrival_order(g, name, M, N, K, plan):
    # fp32 partial sums of a k split are added in split order by whichever
    # block of the tile arrives last, so repeated calls give the same fp16
    # bits (and match the oracle like any plan)
    op = getattr(g, "W4_OP_" + name.upper())
    s = Shape(g, op, M, N, K, seed=14000 + M)
    names = [g.w4_plan_name(op, M, N, K, i) for i in range(g.w4_plan_count(op, M, N, K))]
    assert plan in names
    say(f"case repeat {name} M={M} N={N} K={K} {plan}")
    try:
        g.w4_plan_pin(op, M, N, K, names.index(plan))
        outs = [s.run(g.W4_OUT_F16, bias=True) for _ in range(4)]
        for o in outs[1:]:
            assert np.array_equal(o.view(np.uint16), outs[0].view(np.uint16))
        s.check(f"{name} {M}x{N}x{K} {plan}")
    finally:
        g.w4_plan_pin(op, M, N, K, -1)


@pytest.mark.parametrize("name,M,N,K,plan", [
    ("w4a8", 300, 2000, 1040, "gemm:128x256"),
    ("w2a8", 1100, 2000, 1024, "gemm:128x128,ksplit=2"),
    ("w4a16", 16, 1024, 4096, "skinny:ksplit=4"),
    ("w2a8", 128, 3200, 3200, "skinny:rows=32,ksplit=2"),
    ("w4a16", 4, 4096, 11008, "decode:ksplit=4"),
    ("w2a8", 1, 8640, 3200, "decode:ksplit=1,waves=4"),
    ("w4a16", 16, 4096, 4096, "decode:ksplit=1,waves=16"),
])
def test_graph_replays_match_eager(g, name, M, N, K, plan):
    # The GEMM, the skinny kernel and the decode kernel (split, and with 4 and
    # 16 waves per block) are captured in a HIP graph and replayed three
    # times with eager work in between; each replay must give the eager
    # call's output bit for bit (split counters are left zero by each call,
    # no memset is recorded).
    op = getattr(g, "W4_OP_" + name.upper())
    s = Shape(g, op, M, N, K, seed=15000 + M)
    names = [g.w4_plan_name(op, M, N, K, i) for i in range(g.w4_plan_count(op, M, N, K))]
    assert plan in names
    say(f"case graph {name} M={M} N={N} K={K} {plan}")
    try:
        g.w4_plan_pin(op, M, N, K, names.index(plan))
        need = g.w4_plan_workspace_bytes(op, M, N, K)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda") if need else None
        if op == g.W4_OP_W4A16:
            C = torch.empty((M, N), dtype=torch.float16, device="cuda")
            A = dev(s.A)
            call = lambda: g.w4a16_gemm(A, s.Wp, N, workspace=ws, C=C)
        else:
            C = torch.empty((M, N), dtype=torch.int32, device="cuda")
            mm = g.w4a8_gemm if op == g.W4_OP_W4A8 else g.w2a8_gemm
            call = lambda: mm(s.Aq, s.sa, s.Wp, s.scale, N, out_dtype=g.W4_OUT_I32,
                              workspace=ws, C=C)
        call()
        eager = host(C).copy()
        # the eager output itself against the oracle, every element
        if op == g.W4_OP_W4A16:
            tol_ok(eager, s.ref_f16(bias=False), f"graph eager {plan}")
        else:
            assert np.array_equal(eager, s.acc.astype(np.int32)), plan
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        for rep in range(3):
            C.fill_(0)                                  # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            got = host(C)
            assert np.array_equal(got.view(np.uint8), eager.view(np.uint8)), rep
            # and each replay against the oracle directly
            if op == g.W4_OP_W4A16:
                tol_ok(got, s.ref_f16(bias=False), f"graph replay {rep} {plan}")
            else:
                assert np.array_equal(got, s.acc.astype(np.int32)), (rep, plan)
        if need:
            assert not host(ws[:16384]).any()           # counters zero after the replays
    finally:
        g.w4_plan_pin(op, M, N, K, -1)


def _random_shapes():
    # two ragged shapes per kind from one fixed seed: rows 1..16 and
    # 17..140, columns 1..700 (partial n-tiles), K a required multiple up to
    # 4096 (k tails)
    rng = np.random.default_rng(16000)
    out = []
    for name, kmult in (("w4a8", 16), ("w2a8", 16), ("w4a16", 128), ("w2a16", 16),
                        ("w8a8", 16), ("f8f8", 16)):
        for lo, hi in ((1, 17), (17, 141)):
            M = int(rng.integers(lo, hi))
            N = int(rng.integers(1, 701))
            K = int(rng.integers(1, 4096 // kmult + 1)) * kmult
            out.append((name, M, N, K))
    return out


@pytest.mark.parametrize("name,M,N,K", _random_shapes())
def test_random_shapes_every_plan(g, name, M, N, K):
    test_every_plan_matches_oracle(g, name, M, N, K)


def test_split_plans_on_a_side_stream(g):
    # Split plans launched on a stream other than the current one, without
    # switching the current stream: the wrapper's temporary workspace must be
    # zero-filled on the launch stream (not on the current one), and a shared
    # Workspace first used on the current stream must be ordered before the
    # side-stream call. Every result against the oracle, every element.
    op, M, N, K = g.W4_OP_W2A8, 1, 16, 131056
    s = Shape(g, op, M, N, K, seed=17000)
    assert g.w4_plan_name(op, M, N, K, g.w4_plan_current(op, M, N, K)) == "decode:ksplit=64"
    s16 = Shape(g, g.W4_OP_W4A16, 1, 512, 8192, seed=17100)
    names = [g.w4_plan_name(g.W4_OP_W4A16, 1, 512, 8192, i)
             for i in range(g.w4_plan_count(g.W4_OP_W4A16, 1, 512, 8192))]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    say("case side stream: w2a8 decode:ksplit=64 and w4a16 decode:ksplit=4, fresh workspaces")
    try:
        g.w4_plan_pin(g.W4_OP_W4A16, 1, 512, 8192, names.index("decode:ksplit=4"))
        A16 = dev(s16.A)
        torch.cuda.synchronize()
        for rep in range(3):
            # busy the current stream so that unordered work would overlap
            junk = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
            junk.fill_(0xFF)
            C = g.w2a8_gemm(s.Aq, s.sa, s.Wp, s.scale, N, out_dtype=g.W4_OUT_I32, stream=side)
            C16 = g.w4a16_gemm(A16, s16.Wp, 512, stream=side)
            side.synchronize()
            assert np.array_equal(C.cpu().numpy(), s.acc.astype(np.int32)), rep
            tol_ok(C16.cpu().numpy(), s16.ref_f16(bias=False), f"side stream w4a16 {rep}")
            del junk
        say("case side stream: one Workspace used on the current stream, then on a side stream")
        ws = g.Workspace("cuda")
        Ccur = g.w2a8_gemm(s.Aq, s.sa, s.Wp, s.scale, N, out_dtype=g.W4_OUT_I32, workspace=ws)
        Cside = g.w2a8_gemm(s.Aq, s.sa, s.Wp, s.scale, N, out_dtype=g.W4_OUT_I32, workspace=ws,
                            stream=side)
        side.synchronize()
        torch.cuda.synchronize()
        assert np.array_equal(Ccur.cpu().numpy(), s.acc.astype(np.int32))
        assert np.array_equal(Cside.cpu().numpy(), s.acc.astype(np.int32))
        assert not ws.buf[:16384].cpu().numpy().any()
    finally:
        g.w4_plan_pin(g.W4_OP_W4A16, 1, 512, 8192, -1)
