"""GPU parity: every kernel through the C ABI against the CPU oracle.

Bit-exact for packed bytes, scales, zeros, INT8 activations and INT32
accumulators; |gpu - ref| <= 2^-9 |ref| + 1e-3 rms(ref) for fp16/fp32 outputs.
"""
import numpy as np
import pytest

import oracle as O
from gemv_nibble_unpack_amd import workloads as WL
from tests._helpers import say, sample_indices, tol_ok

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemv_nibble_unpack_amd as G
    G.load()
    return G


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def f16(x):
    return dev(np.asarray(x, np.float16))


# ---------------------------------------------------------------------------
# offline weight preparation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,K", [(256, 256), (50, 96), (11008, 4096)])
def test_quantize_pack_w4_sym_bitexact(g, N, K):
    say(f"case quantize_pack_w4 sym N={N} K={K}")
    W = WL.weights_f32(N, K, seed=1000 + N + K)
    W[3 % N, :] = 0.0                                  # a zero row
    Wq, s, z = g.quantize_pack_w4(dev(W), g.W4_SYM_PER_CHANNEL)
    q_ref, s_ref = O.quantize_w4_sym(W)
    assert z is None
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(Wq), O.pack_int4(q_ref))


@pytest.mark.parametrize("N,K", [(4096, 4096), (11008, 4096), (4096, 11008), (37, 256)])
def test_quantize_pack_w4_group_bitexact(g, N, K):
    say(f"case quantize_pack_w4 group N={N} K={K}")
    W = WL.weights_f32(N, K, seed=2000 + N + K)
    W[0, :128] = 0.25                                  # constant group -> scale 0
    W[min(1, N - 1), 128:256] = np.linspace(1.0, 2.0, 128, dtype=np.float32)  # clipped zero
    Wq, s, z = g.quantize_pack_w4(dev(W), g.W4_ASYM_GROUP)
    q_ref, s_ref, z_ref = O.quantize_w4_group(W, 128)
    assert np.array_equal(host(s).view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(host(z), z_ref)
    assert np.array_equal(host(Wq), O.pack_int4(q_ref))


@pytest.mark.parametrize("N,K", [(3200, 3200), (8640, 3200), (3200, 8640), (5, 20)])
def test_quantize_pack_w2_and_scale(g, N, K):
    say(f"case quantize_pack_w2 N={N} K={K}")
    codes = WL.ternary_codes(N, K, seed=3000 + N + K)
    src = WL.weights_f32(N, K, seed=3001 + N + K)
    Wq = g.quantize_pack_w2(dev(codes))
    assert np.array_equal(host(Wq), O.pack_int2(codes))
    s = host(g.ternary_scale_f16(dev(src)))[0]
    ref = O.ternary_scale(src)
    # both sides round a float64 mean once to fp16; they may differ only if
    # the mean sits within float64 summation noise of an fp16 midpoint
    mean = np.abs(src.astype(np.float64)).sum() / src.size
    lo, hi = np.float16(mean * (1 - 1e-12)), np.float16(mean * (1 + 1e-12))
    assert s == ref or (lo != hi and s in (lo, hi))


@pytest.mark.parametrize("M,K,dt", [(1, 256, np.float32), (2048, 4096, np.float16),
                                    (3, 8, np.float16), (17, 1000, np.float32),
                                    (5, 8192, np.float16), (3, 11008, np.float16),
                                    (6, 8200, np.float32)])
def test_quantize_a8_bitexact(g, M, K, dt):
    say(f"case quantize_a8 M={M} K={K} {dt.__name__}")
    A = WL.activations(M, K, seed=4000 + M + K, dtype=dt)
    A[M // 2, :] = 0
    Aq, sa, rs = g.quantize_a8(dev(A))
    qa_ref, sa_ref, rs_ref = O.quantize_a8(A)
    assert np.array_equal(host(sa), sa_ref)
    assert np.array_equal(host(Aq), qa_ref)
    assert np.array_equal(host(rs), rs_ref)


def _near_tie_rows(K=2048):
    """Rows whose quotients a / s sit on and next to every half integer: for
    several row maxima, a = fl((k + 1/2) * s) and its float32 neighbours up to
    4 ulp away, so the code decision is taken right at its rounding edges."""
    rows = []
    for amax in (127.0, 100.0, 3.7, 0.013, 6.1e4):
        s = np.float32(np.float32(amax) / np.float32(127.0))
        vals = [np.float32(amax)]
        for k in range(-127, 127):
            x = np.float32((k + 0.5) * np.float64(s))
            for d in range(-4, 5):
                y = x
                step = np.float32(np.inf if d > 0 else -np.inf)
                for _ in range(abs(d)):
                    y = np.nextafter(y, step)
                if abs(y) <= amax:
                    vals.append(y)
        for i in range(0, len(vals), K - 1):
            row = np.zeros(K, np.float32)
            chunk = vals[i:i + K - 1]
            row[0] = np.float32(amax)
            row[1:1 + len(chunk)] = chunk
            rows.append(row)
    return np.stack(rows)


def test_quantize_a8_near_ties(g):
    # the kernel decides codes by a reciprocal multiply and falls back to the
    # division only near half integers; this pins that edge bit-exactly
    A = _near_tie_rows()
    say(f"case quantize_a8 near ties M={A.shape[0]} K={A.shape[1]}")
    Aq, sa, rs = g.quantize_a8(dev(A))
    qa_ref, sa_ref, rs_ref = O.quantize_a8(A)
    assert np.array_equal(host(sa), sa_ref)
    assert np.array_equal(host(Aq), qa_ref)
    assert np.array_equal(host(rs), rs_ref)


def test_quantize_a8_tiny_rows(g):
    # float32 rows whose scale max|a| / 127 is subnormal or just normal: a
    # subnormal scale carries its own rounding error (|a / s| can pass 127, so
    # the clip acts), and its reciprocal can overflow; the codes still follow
    # rint(fl(a / s)) clipped to [-127, 127]. Also without the row sums.
    rng = np.random.default_rng(4100)
    K = 1024
    rows = []
    for amax in (1e-37, 2.0 ** -126 * 127, 2.0 ** -126 * 126.9, 3e-39, 7e-44, 2.0 ** -149 * 5):
        r = (rng.uniform(-1.0, 1.0, K) * amax).astype(np.float32)
        r[rng.integers(0, K)] = np.float32(amax)
        rows.append(r)
    A = np.stack(rows)
    say(f"case quantize_a8 tiny rows M={A.shape[0]} K={K}")
    Aq, sa, rs = g.quantize_a8(dev(A))
    qa_ref, sa_ref, rs_ref = O.quantize_a8(A)
    assert np.array_equal(host(sa), sa_ref)
    assert np.array_equal(host(Aq), qa_ref)
    assert np.array_equal(host(rs), rs_ref)
    Aq2, sa2, _ = g.quantize_a8(dev(A), with_rowsum=False)
    assert np.array_equal(host(Aq2), qa_ref) and np.array_equal(host(sa2), sa_ref)


@pytest.mark.parametrize("layout,N,K", [(0, 256, 256), (0, 50, 208), (1, 4096, 4096),
                                        (1, 37, 384), (2, 3200, 8640), (2, 19, 48)])
def test_prepack_roundtrip(g, layout, N, K):
    say(f"case prepack layout={layout} N={N} K={K}")
    rng = np.random.default_rng(layout * 100 + N)
    rowbytes = K // 4 if layout == 2 else K // 2
    Wq = rng.integers(0, 256, size=(N, rowbytes), dtype=np.uint8)
    s = z = None
    if layout == 1:
        s = dev(rng.random((N, K // 128)).astype(np.float16))
        z = dev(rng.integers(0, 16, size=(N, K // 128), dtype=np.uint8))
    Wp = g.prepack_w(layout, dev(Wq), N, K, s, z)
    assert Wp.numel() == g.prepack_bytes(layout, N, K)
    Wq2, s2, z2 = g.unprepack_w(layout, Wp, N, K)
    assert np.array_equal(host(Wq2), Wq)
    if layout == 1:
        assert np.array_equal(host(s2).view(np.uint16), host(s).view(np.uint16))
        assert np.array_equal(host(z2), host(z))


# ---------------------------------------------------------------------------
# matmul paths
# ---------------------------------------------------------------------------
def prep_w4a8(g, W):
    N, K = W.shape
    Wq, s, _ = g.quantize_pack_w4(dev(W), g.W4_SYM_PER_CHANNEL)
    return g.prepack_w(g.W4_LAYOUT_W4A8, Wq, N, K), s


def prep_w4a16(g, W):
    N, K = W.shape
    Wq, s, z = g.quantize_pack_w4(dev(W), g.W4_ASYM_GROUP)
    return g.prepack_w(g.W4_LAYOUT_W4A16, Wq, N, K, s, z)


def prep_w2a8(g, codes, src):
    N, K = codes.shape
    Wq = g.quantize_pack_w2(dev(codes))
    return g.prepack_w(g.W4_LAYOUT_W2A8, Wq, N, K), g.ternary_scale_f16(dev(src))


def test_w4a8_gemv_tiny_config(g):
    c = WL.W4A8_TINY
    say(f"case {c.name}")
    d = c.inputs()
    Wp, ws = prep_w4a8(g, d["W"])
    Aq, sa, _ = g.quantize_a8(dev(d["A"]))
    q_ref, s_ref = O.quantize_w4_sym(d["W"])
    qa_ref, sa_ref, _ = O.quantize_a8(d["A"])
    acc_ref = O.int_accumulate(qa_ref, q_ref)
    C32 = g.w4a8_gemm(Aq, sa, Wp, ws, c.N, out_dtype=g.W4_OUT_I32)
    assert np.array_equal(host(C32), acc_ref.astype(np.int32))
    Cf = g.w4a8_gemm(Aq, sa, Wp, ws, c.N, out_dtype=g.W4_OUT_F32)
    tol_ok(host(Cf), O.w4a8_gemm(qa_ref, sa_ref, q_ref, s_ref, None, O.OUT_F32), c.name)


@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (1, 50, 208), (3, 100, 1024), (16, 256, 512),
                                   (17, 40, 256), (5, 2048, 11008), (130, 300, 208),
                                   (256, 4096, 1024), (64, 520, 4096)])
def test_w4a8_small_shapes_bitexact(g, M, N, K):
    say(f"case w4a8 M={M} N={N} K={K}")
    W = WL.weights_f32(N, K, seed=5000 + N)
    A = WL.activations(M, K, seed=5001 + M)
    bias = WL.bias_f16(N, seed=5002)
    Wp, ws = prep_w4a8(g, W)
    Aq, sa, _ = g.quantize_a8(dev(A))
    q_ref, s_ref = O.quantize_w4_sym(W)
    qa_ref, sa_ref, _ = O.quantize_a8(A)
    acc = O.int_accumulate(qa_ref, q_ref)
    C32 = g.w4a8_gemm(Aq, sa, Wp, ws, N, out_dtype=g.W4_OUT_I32)
    assert np.array_equal(host(C32), acc.astype(np.int32))
    C16 = g.w4a8_gemm(Aq, sa, Wp, ws, N, bias=f16(bias), out_dtype=g.W4_OUT_F16)
    tol_ok(host(C16).astype(np.float64),
           O.w4a8_gemm(qa_ref, sa_ref, q_ref, s_ref, bias, O.OUT_F16), "f16")


def test_w4a8_prefill_config_full(g):
    # every one of the M x N outputs: INT32 bit for bit, fp16 to the tolerance
    c = WL.W4A8_PREFILL
    say(f"case {c.name}")
    d = c.inputs()
    Wp, ws = prep_w4a8(g, d["W"])
    Aq, sa, _ = g.quantize_a8(dev(d["A"]))
    bias = d["bias"]
    C32 = host(g.w4a8_gemm(Aq, sa, Wp, ws, c.N, out_dtype=g.W4_OUT_I32))
    C16 = host(g.w4a8_gemm(Aq, sa, Wp, ws, c.N, bias=f16(bias), out_dtype=g.W4_OUT_F16))
    q_ref, s_ref = O.quantize_w4_sym(d["W"])
    qa_ref, sa_ref, _ = O.quantize_a8(d["A"])
    assert np.array_equal(host(Aq), qa_ref)
    assert np.array_equal(host(ws), s_ref)
    acc = O.int_accumulate_f64(qa_ref, q_ref)
    assert np.array_equal(C32, acc.astype(np.int32))
    # the float64 route against the int64 sums on a sample
    rows, cols = sample_indices(c.M, c.N, 2000, seed=7)
    assert np.array_equal(acc[rows, cols], O.int_accumulate_entries(qa_ref, q_ref, rows, cols))
    tol_ok(C16, O.dequant_epilogue(acc, s_ref[None, :], sa_ref[:, None], bias[None, :],
                                   O.OUT_F16), c.name)


@pytest.mark.parametrize("scheme,M,N,K", [("w4a8", 2000, 3000, 1040), ("w4a8", 1100, 4004, 512),
                                          ("w4a8", 2000, 11000, 1040), ("w4a8", 1900, 11004, 512),
                                          ("w2a8", 2000, 3000, 1040), ("w2a8", 1030, 4100, 528)])
def test_gemm_path_ragged_full(g, scheme, M, N, K):
    # shapes large enough for the tiled prefill GEMM (>= 128 tiles), with
    # ragged M, N (N % 8 != 0 takes the direct epilogue) and K tails; the
    # N ~ 11000 shapes run 22-tile (352-column) blocks, the others 16 or 8
    say(f"case gemm path {scheme} M={M} N={N} K={K}")
    A = WL.activations(M, K, seed=8000 + M)
    bias = WL.bias_f16(N, seed=8001)
    Aq, sa, _ = g.quantize_a8(dev(A))
    qa, sa_ref, _ = O.quantize_a8(A)
    if scheme == "w4a8":
        W = WL.weights_f32(N, K, seed=8002 + N)
        Wp, ws = prep_w4a8(g, W)
        qw, s_ref = O.quantize_w4_sym(W)
        mm = g.w4a8_gemm
        ws_ref = s_ref[None, :]
    else:
        codes = WL.ternary_codes(N, K, seed=8003 + N)
        Wp, ws = prep_w2a8(g, codes, WL.weights_f32(N, K, seed=8004 + N))
        qw = codes
        mm = g.w2a8_gemm
        ws_ref = np.float64(host(ws)[0])
    C32 = host(mm(Aq, sa, Wp, ws, N, out_dtype=g.W4_OUT_I32))
    C16 = host(mm(Aq, sa, Wp, ws, N, bias=f16(bias), out_dtype=g.W4_OUT_F16))
    C32f = host(mm(Aq, sa, Wp, ws, N, out_dtype=g.W4_OUT_F32))
    acc = O.int_accumulate_f64(qa, qw)
    assert np.array_equal(C32, acc.astype(np.int32))
    tol_ok(C16, O.dequant_epilogue(acc, ws_ref, sa_ref[:, None], bias[None, :], O.OUT_F16), "f16")
    tol_ok(C32f, O.dequant_epilogue(acc, ws_ref, sa_ref[:, None], None, O.OUT_F32), "f32")


def _w4a16_case(g, c, full=True):
    say(f"case {c.name}")
    d = c.inputs()
    Wp = prep_w4a16(g, d["W"])
    C = host(g.w4a16_gemm(dev(d["A"]), Wp, c.N))
    q, s, z = O.quantize_w4_group(d["W"], 128)
    if full:
        ref = O.w4a16_gemm(d["A"], q, s, z, 128)
        tol_ok(C, ref, c.name)
    else:
        rows, cols = sample_indices(c.M, c.N, 2000, seed=8)
        ref = O.w4a16_entries(d["A"], q, s, z, rows, cols, 128)
        tol_ok(C[rows, cols], ref, c.name)


def test_w4a16_decode_config(g):
    _w4a16_case(g, WL.W4A16_DECODE)


@pytest.mark.parametrize("c", WL.W4A16_SWEEP, ids=lambda c: c.name)
def test_w4a16_sweep(g, c):
    _w4a16_case(g, c)


def test_w4a16_bitblas_example_shape(g):
    _w4a16_case(g, WL.BITBLAS_EXAMPLE)


def test_w4a16_prefill_gemm_full(g):
    # M=2048, N=11008, K=4096 with bias: the tiled fp16 GEMM (its built-in
    # block shape); every output against the oracle
    c = WL.W4A16_PREFILL
    say(f"case {c.name}")
    d = c.inputs()
    Wp = prep_w4a16(g, d["W"])
    C = host(g.w4a16_gemm(dev(d["A"]), Wp, c.N, bias=f16(d["bias"])))
    q, s, z = O.quantize_w4_group(d["W"], 128)
    tol_ok(C, O.w4a16_gemm(d["A"], q, s, z, 128, d["bias"]), c.name)


@pytest.mark.parametrize("M,N,K", [(2, 37, 256), (16, 130, 384), (33, 64, 128), (1, 16, 128),
                                   (1030, 4100, 1024), (2000, 3000, 640)])
def test_w4a16_ragged_with_bias(g, M, N, K):
    # decode, skinny and (M >= 1030) the tiled fp16 GEMM's 128 x 256 blocks:
    # N = 4100 has a ragged last column tile and N % 8 != 0 (direct epilogue),
    # N = 3000 goes through the LDS-staged epilogue; both have rows past M
    say(f"case w4a16 ragged M={M} N={N} K={K}")
    W = WL.weights_f32(N, K, seed=6000 + N)
    A = WL.activations(M, K, seed=6001 + M)
    b = WL.bias_f16(N, seed=6002)
    Wp = prep_w4a16(g, W)
    C = host(g.w4a16_gemm(dev(A), Wp, N, bias=f16(b)))
    q, s, z = O.quantize_w4_group(W, 128)
    tol_ok(C, O.w4a16_gemm(A, q, s, z, 128, b), "ragged")


@pytest.mark.parametrize("c", WL.W2A8_TERNARY, ids=lambda c: c.name)
def test_w2a8_ternary(g, c):
    say(f"case {c.name}")
    d = c.inputs()
    Wp, s16 = prep_w2a8(g, d["codes"], d["src"])
    Aq, sa, _ = g.quantize_a8(dev(d["A"]))
    C32 = host(g.w2a8_gemm(Aq, sa, Wp, s16, c.N, out_dtype=g.W4_OUT_I32))
    C16 = host(g.w2a8_gemm(Aq, sa, Wp, s16, c.N, out_dtype=g.W4_OUT_F16))
    qa, sa_ref, _ = O.quantize_a8(d["A"])
    scale = host(s16)[0]
    acc = O.int_accumulate_f64(qa, d["codes"])
    assert np.array_equal(C32, acc.astype(np.int32))
    tol_ok(C16, O.dequant_epilogue(acc, np.float64(scale), sa_ref[:, None], None, O.OUT_F16),
           c.name)


@pytest.mark.parametrize("M,N,K", [(65, 24, 48), (200, 130, 1040), (33, 4100, 256)])
def test_w2a8_ragged_bitexact(g, M, N, K):
    say(f"case w2a8 ragged M={M} N={N} K={K}")
    codes = WL.ternary_codes(N, K, seed=7000 + N)
    src = WL.weights_f32(N, K, seed=7001 + N)
    A = WL.activations(M, K, seed=7002 + M)
    b = WL.bias_f16(N, seed=7003)
    Wp, s16 = prep_w2a8(g, codes, src)
    Aq, sa, _ = g.quantize_a8(dev(A))
    qa, sa_ref, _ = O.quantize_a8(A)
    C32 = host(g.w2a8_gemm(Aq, sa, Wp, s16, N, out_dtype=g.W4_OUT_I32))
    assert np.array_equal(C32, O.int_accumulate(qa, codes).astype(np.int32))
    C16 = host(g.w2a8_gemm(Aq, sa, Wp, s16, N, bias=f16(b), out_dtype=g.W4_OUT_F16))
    tol_ok(C16, O.w2a8_gemm(qa, sa_ref, codes, host(s16)[0], b, O.OUT_F16), "w2a8 ragged")


@pytest.mark.parametrize("kind", ["w4a8", "w2a8", "w8a8"])
def test_extreme_codes_at_max_k_no_overflow(g, kind):
    # The largest products the INT32 accumulators can meet: activation -128
    # (a valid int8 the quantizer never makes) times the most negative stored
    # code (-8 INT4, -2 INT2, -128 INT8; none is made by the quantizers but
    # all decode), summed over the largest K the library accepts: 16384 * K
    # sits just below 2^31. Row 1 mixes in +127 activations and row 1 of the
    # weights the largest positive code, so the sums differ per entry.
    K = g.W4_MAX_K
    N = 16
    say(f"case extreme codes {kind} K={K}")
    qa = np.full((2, K), -128, np.int8)
    qa[1, ::2] = 127
    lo, hi = {"w4a8": (-8, 7), "w2a8": (-2, 1), "w8a8": (-128, 127)}[kind]
    codes = np.full((N, K), lo, np.int8)
    codes[1, 1::3] = hi
    if kind == "w4a8":
        Wq = dev(O.pack_int4(codes))
        layout, mm, scale = g.W4_LAYOUT_W4A8, g.w4a8_gemm, dev(np.ones(N, np.float32))
    elif kind == "w2a8":
        Wq = dev(O.pack_int2(codes))
        layout, mm, scale = g.W4_LAYOUT_W2A8, g.w2a8_gemm, f16(np.ones(1))
    else:
        Wq = dev(codes)
        layout, mm, scale = g.W4_LAYOUT_W8A8, g.w8a8_gemm, dev(np.ones(N, np.float32))
    Wp = g.prepack_w(layout, Wq, N, K)
    C32 = host(mm(dev(qa), dev(np.ones(2, np.float32)), Wp, scale, N, out_dtype=g.W4_OUT_I32))
    ref = O.int_accumulate(qa, codes)
    # the kernels sum 16 q (4-bit), 64 c (2-bit) or the INT8 code as it is:
    # the internal accumulator of entry (0, 0) reaches 16384 K < 2^31
    unpack = {"w4a8": 16, "w2a8": 64, "w8a8": 1}[kind]
    assert ref[0, 0] * unpack == 16384 * K < 2**31
    assert np.array_equal(C32, ref.astype(np.int32))


def test_matmul_m0_is_noop_and_errors(g):
    say("case m0 and error statuses")
    Aq = dev(np.zeros((0, 256), np.int8))
    W = WL.weights_f32(16, 256, seed=1)
    Wp, ws = prep_w4a8(g, W)
    C = g.w4a8_gemm(Aq, dev(np.zeros(0, np.float32)), Wp, ws, 16)
    assert C.shape == (0, 16)
    with pytest.raises(g.W4Error) as e:
        g.w4a16_gemm(f16(np.zeros((1, 256))), Wp, 16, group_size=64)
    assert e.value.status == -4


# ---------------------------------------------------------------------------
# fused activation quantization (quantize_a8 + matmul in one call)
# ---------------------------------------------------------------------------
def test_fused_act_tiny_and_tie_rows(g):
    # the prologue's code rule at its edges: quotients on and next to half
    # integers, and float32 rows with subnormal or just-normal scales; one
    # fused call per row (M=1 decode) against the two-call path
    ties = _near_tie_rows(K=1024)
    rng = np.random.default_rng(4200)
    tiny = []
    for amax in (1e-37, 2.0 ** -126 * 127, 2.0 ** -126 * 126.9, 3e-39):
        r = (rng.uniform(-1.0, 1.0, 1024) * amax).astype(np.float32)
        r[rng.integers(0, 1024)] = np.float32(amax)
        tiny.append(r)
    rows = np.concatenate([ties[::3], np.stack(tiny)])
    N, K = 256, 1024
    Wp, ws = prep_w4a8(g, WL.weights_f32(N, K, seed=4201))
    say(f"case fused act edge rows: {rows.shape[0]} rows N={N} K={K}")
    for m in range(rows.shape[0]):
        Ad = dev(rows[m:m + 1])
        Aq, sa, _ = g.quantize_a8(Ad)
        qa_ref, _, _ = O.quantize_a8(rows[m:m + 1])
        assert np.array_equal(host(Aq), qa_ref), m
        ref = host(g.w4a8_gemm(Aq, sa, Wp, ws, N, out_dtype=g.W4_OUT_I32))
        got = host(g.w4a8_gemm_fused_act(Ad, Wp, ws, N, out_dtype=g.W4_OUT_I32))
        assert np.array_equal(ref, got), m


@pytest.mark.parametrize("scheme,M,N,K,dt", [
    ("w4a8", 1, 256, 256, np.float32),      # the tiny GEMV configuration
    ("w4a8", 1, 4096, 4096, np.float16),
    ("w4a8", 4, 4096, 4096, np.float16),
    ("w4a8", 3, 130, 208, np.float16),      # ragged rows and columns, k tail in the last tile
    ("w4a8", 9, 512, 1024, np.float32),     # more than 8 rows: two rows per wave
    ("w4a8", 1, 256, 4096, np.float16),     # split K: every block reads the whole row
    ("w4a8", 40, 300, 512, np.float16),     # three 16-row tiles through the prologue
    ("w4a8", 1, 4096, 11008, np.float16),   # long rows: several chunks per lane
    ("w4a8", 16, 4096, 4096, np.float16),   # too wide for the prologue: two launches
    ("w4a8", 300, 2000, 1040, np.float16),  # skinny kernel: two launches
    # prefill GEMM shapes: quantize_a8 into the workspace, then the GEMM
    ("w4a8", 2048, 11008, 4096, np.float16),  # 256 x 352 blocks
    ("w4a8", 2000, 3000, 1040, np.float16),   # 128 x 256
    ("w4a8", 1100, 4004, 8208, np.float32),   # float32 rows
    ("w2a8", 1100, 2000, 1024, np.float16),   # split over K
    ("w2a8", 1030, 4100, 8240, np.float32),
    ("w2a8", 1, 3200, 3200, np.float16),
    ("w2a8", 1, 8640, 3200, np.float16),
    ("w2a8", 5, 100, 528, np.float32),
])
def test_fused_act_matches_two_calls_and_oracle(g, scheme, M, N, K, dt):
    say(f"case fused act {scheme} M={M} N={N} K={K} {dt.__name__}")
    A = WL.activations(M, K, seed=9000 + M + K, dtype=dt)
    if M > 2:
        A[1, :] = 0                             # a zero row: scale 0, codes 0, output = bias
    bias = WL.bias_f16(N, seed=9001)
    if scheme == "w4a8":
        W = WL.weights_f32(N, K, seed=9002 + N)
        Wp, ws = prep_w4a8(g, W)
        qw, _ = O.quantize_w4_sym(W)
        mm, fused = g.w4a8_gemm, g.w4a8_gemm_fused_act
    else:
        codes = WL.ternary_codes(N, K, seed=9003 + N)
        Wp, ws = prep_w2a8(g, codes, WL.weights_f32(N, K, seed=9004 + N))
        qw = codes
        mm, fused = g.w2a8_gemm, g.w2a8_gemm_fused_act
    Ad = dev(A)
    Aq, sa, _ = g.quantize_a8(Ad)
    plan = g.w4_plan_name(g.W4_OP_W4A8 if scheme == "w4a8" else g.W4_OP_W2A8, M, N, K,
                          g.w4_plan_current(g.W4_OP_W4A8 if scheme == "w4a8" else g.W4_OP_W2A8,
                                            M, N, K))
    say(f"  plan {plan}")
    for out in (g.W4_OUT_I32, g.W4_OUT_F32, g.W4_OUT_F16):
        b = f16(bias) if out == g.W4_OUT_F16 else None
        ref = host(mm(Aq, sa, Wp, ws, N, bias=b, out_dtype=out))
        got = host(fused(Ad, Wp, ws, N, bias=b, out_dtype=out))
        assert np.array_equal(ref, got), out
        if out == g.W4_OUT_I32:
            qa, _, _ = O.quantize_a8(A)
            assert np.array_equal(got, O.int_accumulate_f64(qa, qw).astype(np.int32))


def test_fused_prefill_shared_workspace_across_calls_and_graphs(g):
    # Fused prefill calls of different shapes in a row through one shared
    # workspace (with a 64-way split decode call between them, whose arrival
    # counters live in the same counter area), and three replays of a
    # captured fused call, all equal their results on fresh workspaces and
    # the oracle.
    cases = [(2000, 3000, 1040, 0), (1100, 2000, 1024, 2), (600, 11000, 1040, 0)]
    ops = []
    for i, (M, N, K, kind) in enumerate(cases):
        A = WL.activations(M, K, seed=9600 + i, dtype=np.float16)
        if kind == 0:
            W = WL.weights_f32(N, K, seed=9610 + i)
            Wp, ws = prep_w4a8(g, W)
            qw, _ = O.quantize_w4_sym(W)
            fn = g.w4a8_gemm_fused_act
        else:
            codes = WL.ternary_codes(N, K, seed=9620 + i)
            Wp, ws = prep_w2a8(g, codes, WL.weights_f32(N, K, seed=9630 + i))
            qw, fn = codes, g.w2a8_gemm_fused_act
        qa, _, _ = O.quantize_a8(A)
        ops.append((dev(A), Wp, ws, N, fn, O.int_accumulate_f64(qa, qw).astype(np.int32)))
    # the split decode call between them
    codes = WL.ternary_codes(16, 131056, seed=9640)
    Wd, wsd = prep_w2a8(g, codes, WL.weights_f32(16, 131056, seed=9641))
    Ad = dev(WL.activations(1, 131056, seed=9642, dtype=np.float16))
    qa, sa_d, _ = O.quantize_a8(host(Ad))
    acc_d = O.int_accumulate_f64(qa, codes).astype(np.int32)
    Aq_d, sa_dd, _ = g.quantize_a8(Ad)
    need = max(g.w4_fused_act_workspace_bytes(g.W4_LAYOUT_W4A8 if kind == 0 else
                                              g.W4_LAYOUT_W2A8, M, N, K)
               for (M, N, K, kind) in cases)
    need = max(need, g.w4_plan_workspace_bytes(g.W4_OP_W2A8, 1, 16, 131056))
    shared = torch.zeros(need, dtype=torch.uint8, device="cuda")
    say(f"case fused prefill: shared workspace of {need} bytes, three shapes and a split call")
    for rep in range(2):
        for i, (A, Wp, ws, N, fn, acc) in enumerate(ops):
            got = host(fn(A, Wp, ws, N, out_dtype=g.W4_OUT_I32, workspace=shared))
            assert np.array_equal(got, acc), (rep, i)
            assert np.array_equal(got, host(fn(A, Wp, ws, N, out_dtype=g.W4_OUT_I32))), (rep, i)
            got = host(g.w2a8_gemm(Aq_d, sa_dd, Wd, wsd, 16, out_dtype=g.W4_OUT_I32,
                                   workspace=shared))
            assert np.array_equal(got, acc_d), (rep, i)
        assert not host(shared[:16384]).any()
    say("case fused prefill: graph capture, three replays")
    A, Wp, ws, N, fn, acc = ops[0]
    C = torch.empty((cases[0][0], N), dtype=torch.int32, device="cuda")
    call = lambda: fn(A, Wp, ws, N, out_dtype=g.W4_OUT_I32, workspace=shared, C=C)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r in range(3):
        C.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        assert np.array_equal(host(C), acc), r
    assert not host(shared[:16384]).any()


# ---------------------------------------------------------------------------
# graph capture of a decode chain (INT4 page, Part 2)
# ---------------------------------------------------------------------------
def test_decode_chain_graph_replays_match_eager(g):
    # A decode step's chain of GEMVs captured once and replayed: fp16 output
    # of one layer feeds the next (4096 -> 11008 -> 4096 -> 4096 -> 3200
    # columns), mixing W4A16, fused W4A8 and fused W2A8 calls, one of them
    # split over K (workspace in use). Each layer's eager output is checked
    # against the oracle applied to the GPU's fp16 input of that layer; each
    # replay, with eager work and a synchronization in between, must equal
    # the eager chain bit for bit.
    say("case decode chain graph capture")
    dims = [4096, 11008, 4096, 256, 3200]
    kinds = ["w4a16", "w4a8", "w4a16", "w2a8"]
    layers, refs = [], []
    for i, kind in enumerate(kinds):
        K, N = dims[i], dims[i + 1]
        W = WL.weights_f32(N, K, seed=9100 + i)
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
            codes = WL.ternary_codes(N, K, seed=9200 + i)
            Wp, ws = prep_w2a8(g, codes, W)
            layers.append((kind, Wp, ws, N))

            def ref_w2a8(x, codes=codes, ws=ws):
                qa, sa, _ = O.quantize_a8(x)
                return O.w2a8_gemm(qa, sa, codes, host(ws)[0], None, O.OUT_F16)
            refs.append(ref_w2a8)
    bufs = [torch.empty((1, d), dtype=torch.float16, device="cuda") for d in dims]
    wss = [g.Workspace("cuda") for _ in layers]
    x0 = dev(WL.activations(1, dims[0], seed=9300, dtype=np.float16))

    def chain():
        for i, (kind, Wp, ws, N) in enumerate(layers):
            if kind == "w4a16":
                g.w4a16_gemm(bufs[i], Wp, N, workspace=wss[i], C=bufs[i + 1])
            elif kind == "w4a8":
                g.w4a8_gemm_fused_act(bufs[i], Wp, ws, N, workspace=wss[i], C=bufs[i + 1])
            else:
                g.w2a8_gemm_fused_act(bufs[i], Wp, ws, N, workspace=wss[i], C=bufs[i + 1])

    bufs[0].copy_(x0)
    chain()
    torch.cuda.synchronize()
    eager = [host(b) for b in bufs[1:]]
    assert all(np.isfinite(e.astype(np.float32)).all() for e in eager)
    ins = [host(bufs[0])] + eager[:-1]
    for i, ref in enumerate(refs):
        tol_ok(eager[i], ref(ins[i]), f"chain layer {i} ({kinds[i]})")
    # warm the workspaces, then capture on a side stream
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain()
    for rep in range(3):
        for b in bufs[1:]:
            b.fill_(0)                          # eager work between replays
        bufs[0].copy_(x0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, b in enumerate(bufs[1:]):
            assert np.array_equal(host(b).view(np.uint16), eager[i].view(np.uint16)), (rep, i)


# ---------------------------------------------------------------------------
# FP16 x INT2 (ternary weights, fp16 activations)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("c", WL.W2A16_TERNARY, ids=lambda c: c.name)
def test_w2a16_ternary(g, c):
    say(f"case {c.name}")
    d = c.inputs()
    Wp, ws = prep_w2a8(g, d["codes"], d["src"])
    scale = host(ws)[0]
    C = host(g.w2a16_gemm(dev(d["A"]), Wp, ws, c.N))
    tol_ok(C, O.w2a16_gemm(d["A"], d["codes"], scale), c.name)


@pytest.mark.parametrize("M,N,K", [(5, 100, 528), (3, 37, 48), (17, 260, 1040), (1, 256, 8640),
                                   (40, 300, 512)])
def test_w2a16_ragged_and_split(g, M, N, K):
    # ragged rows/columns/k tails, 16-row tiles, and a split over K (N=256)
    say(f"case w2a16 M={M} N={N} K={K}")
    A = WL.activations(M, K, seed=9500 + M, dtype=np.float16)
    codes = WL.ternary_codes(N, K, seed=9501 + N)
    bias = WL.bias_f16(N, seed=9502)
    Wp, ws = prep_w2a8(g, codes, WL.weights_f32(N, K, seed=9503))
    scale = host(ws)[0]
    C = host(g.w2a16_gemm(dev(A), Wp, ws, N, bias=f16(bias)))
    tol_ok(C, O.w2a16_gemm(A, codes, scale, bias), f"w2a16 {M}x{N}x{K}")


# ---------------------------------------------------------------------------
# INT8 x INT8 (BitBLAS data-type table), INT8 output re-quantized
# ---------------------------------------------------------------------------
def prep_w8a8(g, W):
    N, K = W.shape
    Wq, s = g.quantize_pack_w8(dev(W))
    return g.prepack_w(g.W4_LAYOUT_W8A8, Wq, N, K), s, Wq


def test_quantize_w8_bitexact_and_prepack_roundtrip(g):
    say("case quantize_pack_w8 300x528")
    W = WL.weights_f32(300, 528, seed=9600)
    W[3, :8] = [127.0, 63.5, -0.5, 2.5, 126.5, -127.0, 0.49, 1.5]    # ties, scale 1
    W[3, 8:] = 0
    W[7, :] = 0
    Wp, s, Wq = prep_w8a8(g, W)
    q_ref, s_ref = O.quantize_w8_sym(W)
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(Wq), q_ref)
    back, _, _ = g.unprepack_w(g.W4_LAYOUT_W8A8, Wp, 300, 528)
    assert np.array_equal(host(back).view(np.int8), q_ref)


@pytest.mark.parametrize("M,N,K", [(1, 256, 256), (4, 4096, 4096), (16, 4096, 4096),
                                   (128, 3200, 3200), (3, 130, 208), (1, 256, 8640),
                                   (40, 300, 512), (300, 2000, 1040), (2048, 4096, 4096),
                                   (1100, 2000, 1040), (1030, 1990, 528)])
def test_w8a8_outputs(g, M, N, K):
    # decode (M <= 16), skinny (M = 128, 300), 16-row-tile (M = 40) and tiled
    # GEMM (M >= 1030: 128 x 128 blocks, N % 8 != 0 through the direct
    # epilogue, K tails of 16 past a 64-k tile) kernels, ragged tails and a
    # split over K; every output compared: INT32 and INT8 bit-exact, f16/f32
    # to the tolerance
    say(f"case w8a8 M={M} N={N} K={K}")
    A = WL.activations(M, K, seed=9700 + M, dtype=np.float16)
    W = WL.weights_f32(N, K, seed=9701 + N)
    bias = WL.bias_f16(N, seed=9702)
    Wp, ws, _ = prep_w8a8(g, W)
    Aq, sa, _ = g.quantize_a8(dev(A))
    qa, sa_ref, _ = O.quantize_a8(A)
    qw, ws_ref = O.quantize_w8_sym(W)
    acc = O.int_accumulate_f64(qa, qw)
    C32 = host(g.w8a8_gemm(Aq, sa, Wp, ws, N, out_dtype=g.W4_OUT_I32))
    assert np.array_equal(C32, acc.astype(np.int32))
    # output scale that saturates the largest few codes
    vmax = float(np.max(np.abs((acc.astype(np.float32) * ws_ref[None, :]) * sa_ref[:, None])))
    so = np.float32(vmax / 100.0)
    C8 = host(g.w8a8_gemm(Aq, sa, Wp, ws, N, out_dtype=g.W4_OUT_I8,
                          out_scale=dev(np.array([so], np.float32))))
    assert np.array_equal(C8, O.requantize_i8(acc, ws_ref[None, :], sa_ref[:, None], so))
    C16 = host(g.w8a8_gemm(Aq, sa, Wp, ws, N, bias=f16(bias), out_dtype=g.W4_OUT_F16))
    tol_ok(C16, O.dequant_epilogue(acc, ws_ref[None, :], sa_ref[:, None], bias[None, :],
                                   O.OUT_F16), "f16")
    C32f = host(g.w8a8_gemm(Aq, sa, Wp, ws, N, out_dtype=g.W4_OUT_F32))
    tol_ok(C32f, O.dequant_epilogue(acc, ws_ref[None, :], sa_ref[:, None], None, O.OUT_F32),
           "f32")


# ---------------------------------------------------------------------------
# FP8 E4M3 x FP8 E4M3 (BitBLAS data-type table, last row)
# ---------------------------------------------------------------------------
def _e4m3_tie_row(K=2048):
    """A row whose max is 448 (scale exactly 1, so x / s = x): every midpoint
    between neighbouring E4M3 magnitudes, its float32 neighbours, the exact
    grid values, subnormal ties, both signs, and -0.0."""
    pos = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals = [np.float32(448.0), np.float32(-0.0)]
    for m in mids:
        vals += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))]
    vals += list(pos.astype(np.float32))
    vals += [-v for v in vals[2:]]
    row = np.zeros(K, np.float32)
    row[:len(vals)] = vals[:K]
    return row


@pytest.mark.parametrize("R,K,dt", [(5, 2048, np.float32), (3, 4096, np.float16),
                                    (300, 528, np.float32), (1, 16, np.float16)])
def test_quantize_f8_bitexact(g, R, K, dt):
    say(f"case quantize_f8 R={R} K={K} {dt.__name__}")
    X = WL.activations(R, K, seed=9800 + R + K, dtype=np.float32)
    if dt == np.float32:
        X = X * np.float32(0.02)
        if K >= 2048:
            X[0] = _e4m3_tie_row(K)
    X = X.astype(dt)
    X[R // 2] = 0
    Xq, s = g.quantize_f8(dev(X))
    q_ref, s_ref = O.quantize_f8(X)
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(Xq), q_ref)


def test_f8_every_code_through_the_matrix_core(g):
    # one-hot 1.0 rows against every finite code, on either operand: a single
    # exact product per output, so the float32 result is the code's value
    say("case f8f8 code table")
    codes = np.arange(256, dtype=np.uint8)
    codes[np.isnan(O.e4m3_decode(codes))] = 0
    ones = np.ones(256, np.float32)
    eye = np.zeros((256, 256), np.uint8)
    eye[np.arange(256), np.arange(256)] = 0x38                 # 1.0
    W = np.tile(codes, (16, 1))                                # every row holds codes 0..255
    Wp = g.prepack_w(g.W4_LAYOUT_W8A8, dev(W), 16, 256)
    C = host(g.f8f8_gemm(dev(eye), dev(ones), Wp, dev(ones[:16]), 16, out_dtype=g.W4_OUT_F32))
    want = O.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(C, np.tile(want[:, None], (1, 16)))
    # codes on the activation side, identity weights
    A = np.tile(codes, (16, 1))
    Wp = g.prepack_w(g.W4_LAYOUT_W8A8, dev(eye), 256, 256)
    C = host(g.f8f8_gemm(dev(A), dev(ones[:16]), Wp, dev(ones), 256, out_dtype=g.W4_OUT_F32))
    assert np.array_equal(C, np.tile(want[None, :], (16, 1)))


@pytest.mark.parametrize("M,N,K", [(1, 256, 256), (1, 4096, 4096), (16, 4096, 4096),
                                   (128, 3200, 3200), (3, 130, 208), (1, 256, 8640),
                                   (40, 300, 512), (300, 2000, 1040), (2048, 4096, 4096),
                                   (1100, 2000, 1088), (1030, 2055, 1040)])
def test_f8f8_outputs(g, M, N, K):
    # decode (M <= 16), skinny (M = 128, 300) and 16-row-tile (M = 40)
    # kernels, ragged tails and a split over K (N = 256, K = 8640); the tiled
    # GEMM (M = 2048; M = 1100 over an odd count of 64-k weight tiles, whose
    # last 128-k stage has one live half; M = 1030 with ragged rows, columns
    # and a k tail)
    say(f"case f8f8 M={M} N={N} K={K}")
    A = WL.activations(M, K, seed=9900 + M, dtype=np.float16)
    W = WL.weights_f32(N, K, seed=9901 + N)
    bias = WL.bias_f16(N, seed=9902)
    Wq, ws = g.quantize_f8(dev(W))
    Wp = g.prepack_w(g.W4_LAYOUT_W8A8, Wq, N, K)
    Aq, sa = g.quantize_f8(dev(A))
    qa, sa_ref = O.quantize_f8(A)
    qw, ws_ref = O.quantize_f8(W)
    assert np.array_equal(host(Aq), qa) and np.array_equal(host(Wq), qw)
    C16 = host(g.f8f8_gemm(Aq, sa, Wp, ws, N, bias=f16(bias), out_dtype=g.W4_OUT_F16))
    tol_ok(C16, O.f8f8_gemm(qa, sa_ref, qw, ws_ref, bias, O.OUT_F16), "f16")
    C32 = host(g.f8f8_gemm(Aq, sa, Wp, ws, N, out_dtype=g.W4_OUT_F32))
    tol_ok(C32, O.f8f8_gemm(qa, sa_ref, qw, ws_ref, None, O.OUT_F32), "f32")
