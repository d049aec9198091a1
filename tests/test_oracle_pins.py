"""Pins for the CPU oracle: closed forms, exhaustive tables, brute force,
special cases and the numbers the pages print. CPU only (no GPU marker)."""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
from gemv_nibble_unpack_amd import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def facts():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# symmetric INT4 weights (INT4 page, Part 1 step 1)
# ---------------------------------------------------------------------------
def test_sym_tie_row_half_even_and_range_7():
    # Max 7 -> scale exactly 1 under the /7 reading; halves round to even.
    W = np.array([[7.0, 3.5, 2.5, -0.5, 0.5, 1.5],
                  [7 / 8, 3.5 / 8, 2.5 / 8, -0.5 / 8, 0.5 / 8, 1.5 / 8]], np.float32)
    q, s = O.quantize_w4_sym(W)
    assert s.dtype == np.float32
    assert s.tolist() == [1.0, 0.125]
    assert q.tolist() == [[7, 4, 2, 0, 0, 2]] * 2


def test_sym_negative_max_and_zero_row():
    W = np.array([[-7.0, 1.0, -3.5, 0.0], [0, 0, 0, 0]], np.float32)
    q, s = O.quantize_w4_sym(W)
    assert s.tolist() == [1.0, 0.0]
    assert q.tolist() == [[-7, 1, -4, 0], [0, 0, 0, 0]]


def test_sym_closed_forms_random():
    W = WL.weights_f32(64, 512, seed=11)
    q, s = O.quantize_w4_sym(W)
    amax = np.abs(W).max(axis=1)
    # the largest magnitude maps to +-7, and 7*s reproduces max|w| to 1 ulp
    idx = np.abs(W).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(64), idx]) == 7)
    assert np.all(np.abs(7 * s.astype(np.float64) - amax) <= np.spacing(amax))
    assert q.min() >= -7 and q.max() <= 7
    # every element reconstructs to within half a step (plus float32 slack)
    err = np.abs(W.astype(np.float64) - q * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 2**-20))


# ---------------------------------------------------------------------------
# packing (INT4 page step 1 storage; BitBLAS memory list)
# ---------------------------------------------------------------------------
def test_int4_pack_exhaustive_roundtrip():
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    assert np.array_equal(O.pack_int4(O.unpack_int4(b, signed=True)), b)
    assert np.array_equal(O.pack_int4(O.unpack_int4(b, signed=False)), b)
    # decode by hand for every byte: low nibble first
    s = O.unpack_int4(b, signed=True)[0]
    u = O.unpack_int4(b, signed=False)[0]
    for v in range(256):
        lo, hi = v & 15, v >> 4
        assert u[2 * v] == lo and u[2 * v + 1] == hi
        assert s[2 * v] == (lo - 16 if lo >= 8 else lo)
        assert s[2 * v + 1] == (hi - 16 if hi >= 8 else hi)


def test_int4_pack_spot_values():
    assert O.pack_int4(np.array([[1, -1]])).tolist() == [[0xF1]]
    assert O.pack_int4(np.array([[-7, 7]])).tolist() == [[0x79]]
    assert O.pack_int4(np.array([[15, 0, 3, 12]])).tolist() == [[0x0F, 0xC3]]


def test_int2_pack_exhaustive_and_spot():
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    c = O.unpack_int2(b)
    assert np.array_equal(O.pack_int2(c), b)
    assert c.min() == -2 and c.max() == 1
    assert O.pack_int2(np.array([[1, 0, -1, 0]])).tolist() == [[0b00110001]]
    assert O.pack_int2(np.array([[-1, -1, -1, -1]])).tolist() == [[0xFF]]


def test_packed_sizes_match_page_memory_savings():
    f = facts()["memory_saving_vs_fp16"]
    N, K = 48, 256
    fp16_bytes = N * K * 2
    w4 = O.pack_int4(np.zeros((N, K), np.int8))
    w2 = O.pack_int2(np.zeros((N, K), np.int8))
    assert w4.nbytes == N * K // 2 and w2.nbytes == N * K // 4
    assert 1 - w4.nbytes / fp16_bytes == pytest.approx(f["int4"], abs=0)
    assert 1 - w2.nbytes / fp16_bytes == pytest.approx(f["int2"], abs=0)


# ---------------------------------------------------------------------------
# group-128 asymmetric uINT4 (BitBLAS "Advanced features 2")
# ---------------------------------------------------------------------------
def _grid_group(codes, z0, step):
    return ((np.asarray(codes, np.float64) - z0) * step).astype(np.float32)


def test_group_exact_grid_recovers_codes():
    g = facts()["group_quantization"]["group_size"]
    assert g == 128
    rng = np.random.default_rng(5)
    step = 2.0 ** -6
    codes = rng.integers(0, 16, size=(3, 256))
    codes[:, 0] = 0
    codes[:, 1] = 15          # range covers the whole code space
    codes[:, 128] = 0
    codes[:, 129] = 15
    z0 = np.array([5, 0, 15])
    W = np.stack([_grid_group(codes[i], z0[i], step) for i in range(3)])
    q, s, z = O.quantize_w4_group(W, g)
    assert s.dtype == np.float16 and s.shape == (3, 2) and z.shape == (3, 2)
    assert np.all(s.astype(np.float64) == step)
    assert z[:, 0].tolist() == z0.tolist() and z[:, 1].tolist() == z0.tolist()
    assert np.array_equal(q, codes.astype(np.uint8))


def test_group_tie_rounds_half_even():
    step = 2.0 ** -4
    codes = np.zeros(128)
    codes[:16] = np.arange(16)
    W = _grid_group(codes, 5, step)[None, :]
    W[0, 20] = np.float32(-2.5 * step)   # w/s = -2.5 -> -2 (half-even), +5 -> 3
    W[0, 21] = np.float32(1.5 * step)    # 1.5 -> 2, +5 -> 7
    q, s, z = O.quantize_w4_group(W, 128)
    assert z[0, 0] == 5
    assert q[0, 20] == 3 and q[0, 21] == 7


def test_group_clipped_zero_and_constant_group():
    # all-positive group: min > 0 -> rint(-min/s) < 0 clips to z = 0
    W = np.linspace(1.0, 2.5, 128, dtype=np.float32)[None, :]
    q, s, z = O.quantize_w4_group(W, 128)
    assert z[0, 0] == 0 and q.max() == 15
    # constant group: scale 0 -> codes and zero 0
    q, s, z = O.quantize_w4_group(np.full((1, 128), 0.3, np.float32), 128)
    assert s[0, 0] == 0 and z[0, 0] == 0 and q.max() == 0


def test_group_invariants_random():
    W = WL.weights_f32(32, 1024, seed=12)
    q, s, z = O.quantize_w4_group(W, 128)
    assert q.max() <= 15 and z.max() <= 15
    sf = s.astype(np.float64)
    d = (q.reshape(32, 8, 128).astype(np.float64) - z[:, :, None]) * sf[:, :, None]
    err = np.abs(d.reshape(32, 1024) - W)
    # half a step, plus the slack from using the fp16-rounded scale over <= 15 steps
    s32 = (W.reshape(32, 8, 128).max(2) - W.reshape(32, 8, 128).min(2)) / 15.0
    bound = sf * 0.5 + 16 * np.abs(s32 - sf) + 1e-9
    assert np.all(err.reshape(32, 8, 128) <= bound[:, :, None])


# ---------------------------------------------------------------------------
# INT8 activations (INT4 page, Part 1 step 2)
# ---------------------------------------------------------------------------
def test_a8_ties_range_and_rowsum():
    r = facts()["int8_symmetric_range"]
    A = np.array([[127.0, 63.5, 62.5, -0.5, 0.5, -127.0],
                  [0, 0, 0, 0, 0, 0]], np.float32)
    qa, sa, rs = O.quantize_a8(A)
    assert sa.tolist() == [1.0, 0.0]
    assert qa.tolist() == [[127, 64, 62, 0, 0, -127], [0] * 6]
    assert rs.tolist() == [126, 0]
    A = WL.activations(16, 384, seed=13)
    qa, sa, rs = O.quantize_a8(A)
    assert qa.min() >= r["lo"] and qa.max() <= r["hi"]
    idx = np.abs(A.astype(np.float32)).argmax(axis=1)
    assert np.all(np.abs(qa[np.arange(16), idx]) == 127)
    assert np.array_equal(rs, qa.astype(np.int64).sum(1))


# ---------------------------------------------------------------------------
# integer accumulation and epilogue (INT4 page steps 3-4; BitBLAS statement)
# ---------------------------------------------------------------------------
def _bytes_to_codes_by_hand(byte_rows, bits):
    """Independent slow decoder (pure Python) for the brute-force pin."""
    out = []
    per = 8 // bits
    mask = (1 << bits) - 1
    half = 1 << (bits - 1)
    for row in byte_rows:
        r = []
        for b in row.tolist():
            for i in range(per):
                v = (b >> (bits * i)) & mask
                r.append(v - (1 << bits) if v >= half else v)
        out.append(r)
    return out


@pytest.mark.parametrize("bits", [4, 2])
def test_accumulate_bruteforce_tiny(bits):
    rng = np.random.default_rng(20 + bits)
    M, N, K = 3, 5, 16
    qa = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    if bits == 4:
        codes = rng.integers(-7, 8, size=(N, K))
        packed = O.pack_int4(codes)
        oracle_codes = O.unpack_int4(packed, signed=True)
    else:
        codes = rng.integers(-1, 2, size=(N, K))
        packed = O.pack_int2(codes)
        oracle_codes = O.unpack_int2(packed)
    hand = _bytes_to_codes_by_hand(packed, bits)
    acc = O.int_accumulate(qa, oracle_codes)
    for m in range(M):
        for n in range(N):
            s = 0
            for k in range(K):
                s += int(qa[m, k]) * hand[n][k]
            assert acc[m, n] == s


def test_dp4a_formula_from_page():
    d = facts()["dp4a_example"]
    acc = O.int_accumulate(np.array([d["a"]]), np.array([d["b"]]))
    assert d["c0"] + int(acc[0, 0]) == d["c"]


def test_one_hot_rows_pick_weight_columns_nt():
    rng = np.random.default_rng(7)
    N, K = 6, 10
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    qa = np.zeros((K, K), np.int8)
    qa[np.arange(K), np.arange(K)] = 1
    acc = O.int_accumulate(qa, qw)          # [K, N]
    assert np.array_equal(acc, qw.T.astype(np.int64))


def test_extreme_accumulator_value():
    K = 4096
    acc = O.int_accumulate(np.full((1, K), 127, np.int8), np.full((1, K), 7, np.int8))
    assert acc[0, 0] == 889 * K
    acc = O.int_accumulate(np.full((1, K), -127, np.int8), np.full((1, K), 7, np.int8))
    assert acc[0, 0] == -889 * K


def test_f64_accumulate_equals_int64_random_and_extreme():
    # the float64 product of the codes is the int64 sum exactly: random
    # INT4, INT2 and INT8 codes on ragged shapes, and the extreme products
    # (-128 x -8, -128 x -2, -128 x -128) summed over the largest K the
    # library accepts, where the int32 result sits just below 2^31
    rng = np.random.default_rng(31)
    for (M, N, K, lo, hi) in [(7, 13, 48, -8, 8), (33, 17, 1040, -2, 2), (5, 9, 4096, -128, 128),
                              (64, 80, 528, -128, 128)]:
        qa = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        qw = rng.integers(lo, hi, size=(N, K)).astype(np.int8)
        assert np.array_equal(O.int_accumulate_f64(qa, qw), O.int_accumulate(qa, qw))
    K = 131056
    qa = np.full((2, K), -128, np.int8)
    qa[1, ::2] = 127
    for code in (-8, -2, -128):
        qw = np.full((3, K), code, np.int8)
        qw[1, 1::3] = 7 if code == -8 else 1 if code == -2 else 127
        f = O.int_accumulate_f64(qa, qw)
        assert np.array_equal(f, O.int_accumulate(qa, qw))
    assert O.int_accumulate_f64(np.full((1, K), -128, np.int8),
                                np.full((1, K), -128, np.int8))[0, 0] == 16384 * K
    assert 16384 * K < 2**31 <= 16384 * (K + 16)


def test_f64_accumulate_refuses_rounding_range():
    with pytest.raises(OverflowError):
        O.int_accumulate_f64(np.full((1, 2**20), 127, np.int32), np.full((1, 2**20), 2**30, np.int64))


def test_epilogue_exact_powers_of_two_and_bias():
    acc = np.array([[3, -5], [1000, 7]], np.int64)
    ws = np.array([0.5, 2.0], np.float32)
    sa = np.array([4.0, 0.25], np.float32)
    bias = np.array([1.0, -2.0], np.float16)
    f32 = O.dequant_epilogue(acc, ws[None, :], sa[:, None], None, O.OUT_F32)
    assert f32.tolist() == [[6.0, -40.0], [125.0, 3.5]]
    f16 = O.dequant_epilogue(acc, ws[None, :], sa[:, None], bias[None, :], O.OUT_F16)
    assert f16.dtype == np.float16 and f16.tolist() == [[7.0, -42.0], [126.0, 1.5]]
    assert O.dequant_epilogue(acc, ws, sa, None, O.OUT_I32).tolist() == acc.tolist()


def test_w4a8_zero_activation_row_gives_bias():
    W = WL.weights_f32(8, 64, seed=3)
    q, s = O.quantize_w4_sym(W)
    bias = WL.bias_f16(8, seed=4)
    qa, sa, _ = O.quantize_a8(np.zeros((2, 64), np.float32))
    C = O.w4a8_gemm(qa, sa, q, s, bias, O.OUT_F16)
    assert np.array_equal(C, np.stack([bias, bias]))


def test_w4a8_fp32_matches_float_reference_within_quantisation():
    # end-to-end sanity: the dequantised product approximates the float one
    W = WL.weights_f32(64, 256, seed=31)
    A = WL.activations(1, 256, seed=32, dtype=np.float32)
    q, s = O.quantize_w4_sym(W)
    qa, sa, _ = O.quantize_a8(A)
    C = O.w4a8_gemm(qa, sa, q, s, None, O.OUT_F32).astype(np.float64)
    ref = A.astype(np.float64) @ W.T.astype(np.float64)
    rel = np.linalg.norm(C - ref) / np.linalg.norm(ref)
    assert rel < 0.15


def test_w2a8_scale_and_codes():
    rng = np.random.default_rng(9)
    codes = WL.ternary_codes(4, 64, seed=10)
    assert set(np.unique(codes).tolist()) <= {-1, 0, 1}
    qa = rng.integers(-127, 128, size=(2, 64)).astype(np.int8)
    sa = np.array([1.0, 0.5], np.float32)
    C = O.w2a8_gemm(qa, sa, codes, np.float16(0.25), None, O.OUT_F32)
    acc = qa.astype(np.int64) @ codes.astype(np.int64).T
    assert np.array_equal(C, (acc * 0.25 * sa[:, None]).astype(np.float32))


def test_ternary_scale_exact_sum():
    src = WL.weights_f32(40, 96, seed=14)
    exact = math.fsum(abs(float(x)) for x in src.ravel()) / src.size
    assert O.ternary_scale(src) == np.float16(exact)
    assert O.ternary_scale(np.full((3, 4), -0.375, np.float32)) == np.float16(0.375)


def test_ternary_code_frequencies():
    c = WL.ternary_codes(300, 300, seed=15)
    frac0 = float(np.mean(c == 0))
    assert abs(frac0 - 1 / 3) < 0.01


# ---------------------------------------------------------------------------
# W4A16 (BitBLAS FP16 x INT4 with group scales/zeros)
# ---------------------------------------------------------------------------
def test_w4a16_one_hot_gives_dequantised_weights():
    W = WL.weights_f32(16, 256, seed=16)
    q, s, z = O.quantize_w4_group(W, 128)
    A = np.zeros((256, 256), np.float16)
    A[np.arange(256), np.arange(256)] = 1
    C = O.w4a16_gemm(A, q, s, z, 128)           # [K, N]
    g = np.arange(256) // 128
    deq = (q.astype(np.float64) - z[:, g]) * s[:, g].astype(np.float64)
    assert np.array_equal(C, deq.T.astype(np.float16))


def test_w4a16_zero_point_equal_codes_gives_bias():
    q = np.full((8, 256), 9, np.uint8)
    z = np.full((8, 2), 9, np.uint8)
    s = np.full((8, 2), 0.5, np.float16)
    A = WL.activations(3, 256, seed=17)
    b = WL.bias_f16(8, seed=18)
    C = O.w4a16_gemm(A, q, s, z, 128, b)
    assert np.array_equal(C, np.broadcast_to(b, (3, 8)))


def test_w4a16_bruteforce_groupwise_tiny():
    rng = np.random.default_rng(19)
    M, N, K, g = 2, 3, 256, 128
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    z = rng.integers(0, 16, size=(N, K // g)).astype(np.uint8)
    s = (rng.random((N, K // g)) * 0.01 + 0.001).astype(np.float16)
    A = WL.activations(M, K, seed=21)
    C = O.w4a16_gemm(A, q, s, z, g)
    for m in range(M):
        for n in range(N):
            tot = 0.0
            for gi in range(K // g):
                part = 0.0
                for k in range(gi * g, (gi + 1) * g):
                    part += float(A[m, k]) * (int(q[n, k]) - int(z[n, gi]))
                tot += float(s[n, gi]) * part
            assert abs(float(C[m, n]) - tot) <= abs(tot) * 2**-11 + 1e-7


def test_sampled_entries_agree_with_full():
    rng = np.random.default_rng(22)
    W = WL.weights_f32(40, 256, seed=23)
    A = WL.activations(5, 256, seed=24)
    q4, s4 = O.quantize_w4_sym(W)
    qa, sa, _ = O.quantize_a8(A)
    rows = rng.integers(0, 5, 50)
    cols = rng.integers(0, 40, 50)
    full = O.int_accumulate(qa, q4)
    assert np.array_equal(O.int_accumulate_entries(qa, q4, rows, cols), full[rows, cols])
    qg, sg, zg = O.quantize_w4_group(W, 128)
    full16 = O.w4a16_gemm(A, qg, sg, zg, 128)
    e16 = O.w4a16_entries(A, qg, sg, zg, rows, cols, 128)
    assert np.array_equal(e16, full16[rows, cols])


def test_page_example_shape_is_a_workload():
    ex = facts()["example_matmul_config"]
    c = WL.BITBLAS_EXAMPLE
    assert (c.M, c.N, c.K) == (ex["M"], ex["N"], ex["K"])
    assert ex["layout"] == "nt" and ex["W_dtype"] == "int4"


def test_group_codes_use_fp16_rounded_scale():
    # fp32 scale 2^-6 + 2^-18 rounds to the fp16 scale 2^-6; an element at
    # 7.5 fp16-steps rounds (half-even) to 8 with the fp16 scale but to 7
    # with the unrounded one, so this pins "later steps use the fp16 scale".
    s16 = 2.0 ** -6
    s32 = s16 + 2.0 ** -18
    W = np.zeros((1, 128), np.float32)
    W[0, 0] = -5 * s16
    W[0, 1] = np.float32(-5 * s16 + 15 * s32)
    W[0, 2] = np.float32(2.5 * s16)             # 2.5 steps -> 2 (half-even), +z -> 7
    W[0, 3] = np.float32(7.5 * s16)
    assert np.float32(W[0, 1] - W[0, 0]) / np.float32(15) == np.float32(s32)
    q, s, z = O.quantize_w4_group(W, 128)
    assert float(s[0, 0]) == s16 and z[0, 0] == 5
    assert round(7.5 * s16 / s32) == 7          # the rejected reading
    assert q[0, 3] == 8 + 5
    assert q[0, 2] == 2 + 5                     # 2.5 -> 2 (half-even)


# ---------------------------------------------------------------------------
# FP16 x INT2 (BitBLAS data-type table), on ternary codes (reading 9)
# ---------------------------------------------------------------------------
def test_w2a16_one_hot_rows_pick_scaled_codes():
    rng = np.random.default_rng(31)
    N, K = 7, 48
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    s16 = np.float16(0.015625)                     # 2^-6: products exact
    bias = (rng.normal(0, 0.5, N)).astype(np.float16)
    A = np.zeros((K, K), np.float16)
    A[np.arange(K), np.arange(K)] = 1.0            # row k = e_k
    C = O.w2a16_gemm(A, codes, s16, bias)
    want = (codes.T.astype(np.float64) * 2.0 ** -6 + bias.astype(np.float64)[None, :])
    assert np.array_equal(C, want.astype(np.float16))


def test_w2a16_zero_codes_give_bias_and_negative_codes_subtract():
    A = np.full((2, 32), 2.0, np.float16)
    bias = np.array([0.5, -1.25, 3.0], np.float16)
    C = O.w2a16_gemm(A, np.zeros((3, 32), np.int8), np.float16(0.1), bias)
    assert np.array_equal(C, np.broadcast_to(bias, (2, 3)))
    codes = np.full((3, 32), -1, np.int8)
    C = O.w2a16_gemm(A, codes, np.float16(0.25), None)
    assert np.all(C == np.float16(-16.0))           # 32 * 2 * -1 * 0.25


def test_w2a16_bruteforce_tiny():
    rng = np.random.default_rng(32)
    M, N, K = 3, 5, 64
    A = rng.normal(0, 1, (M, K)).astype(np.float16)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    s16 = np.float16(0.0173)
    bias = rng.normal(0, 0.1, N).astype(np.float16)
    C = O.w2a16_gemm(A, codes, s16, bias)
    for m in range(M):
        for n in range(N):
            acc = math.fsum(float(A[m, k]) * int(codes[n, k]) for k in range(K))
            v = acc * float(s16) + float(bias[n])
            assert C[m, n] == np.float16(v), (m, n)
    rows, cols = np.array([0, 2, 1]), np.array([4, 0, 3])
    assert np.array_equal(O.w2a16_entries(A, codes, s16, rows, cols, bias), C[rows, cols])


# ---------------------------------------------------------------------------
# INT8 x INT8 with INT8 output (BitBLAS data-type table; reading 10)
# ---------------------------------------------------------------------------
def test_w8_page_formula_ties_and_range():
    # the INT4 page's printed formula, /127: max 127 -> scale exactly 1
    W = np.array([[127.0, 63.5, -0.5, 2.5, 126.5, -127.0, 0.49]], np.float32)
    q, s = O.quantize_w8_sym(W)
    assert s.tolist() == [1.0]
    assert q.tolist() == [[127, 64, 0, 2, 126, -127, 0]]
    rng = np.random.default_rng(41)
    W = rng.normal(0, 0.02, (6, 256)).astype(np.float32)
    q, s = O.quantize_w8_sym(W)
    i = np.argmax(np.abs(W), axis=1)
    assert np.all(np.abs(q[np.arange(6), i]) == 127)
    err = np.abs(W.astype(np.float64) - q.astype(np.float64) * s[:, None])
    assert np.all(err <= s[:, None].astype(np.float64) * 0.5 * (1 + 2.0 ** -20))
    q0, s0 = O.quantize_w8_sym(np.zeros((1, 16), np.float32))
    assert s0[0] == 0 and not q0.any()


def test_requantize_i8_exact_cases():
    acc = np.array([[254, -254, 1000, -1000, 5, 0]], np.int64)
    ws = np.array([0.5, 0.5, 0.5, 0.5, 0.5, 0.5], np.float32)
    sa = np.array([1.0], np.float32)
    q = O.requantize_i8(acc, ws[None, :], sa[:, None], 1.0)
    assert q.tolist() == [[127, -127, 127, -127, 2, 0]]         # 2.5 -> 2 (half-even)
    assert not O.requantize_i8(acc, ws[None, :], sa[:, None], 0.0).any()
    # float32 conversion of a large accumulator rounds to nearest even
    big = np.array([[2 ** 24 + 1, 2 ** 24 + 3]], np.int64)
    q = O.requantize_i8(big, np.ones((1, 2), np.float32), np.ones((1, 1), np.float32),
                        2.0 ** 18)
    assert q.tolist() == [[64, 64]]                              # 2^24/2^18, (2^24+4)/2^18


def test_requantize_i8_against_exact_rationals():
    # Independent of the float32 formula: the code is the exact quotient
    # acc * ws * sa / out_scale (the float32 inputs taken as exact binary
    # fractions) rounded half to even and clipped. Three float32 roundings
    # (product, product, quotient; the accumulators stay below 2^24 here, so
    # their conversion is exact) move the quotient by at most 3 * 2^-24 of
    # itself, so the float32 code may differ from the exact one only where the
    # exact quotient lies that close to a half integer, and then only to its
    # other neighbour. A dropped scale, a swapped division or the INT4 /7 or
    # an unscaled clip fails this at once.
    from fractions import Fraction
    rng = np.random.default_rng(4242)
    M, N = 40, 60
    acc = rng.integers(-2 ** 23, 2 ** 23, (M, N)).astype(np.int64)
    ws = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    sa = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
    # an output scale that puts the median |value| near 60: most codes in
    # range, a tail clipped at +-127
    so = np.float32(np.median(np.abs(acc * ws[None, :].astype(np.float64) * sa[:, None])) / 60)
    q = O.requantize_i8(acc, ws[None, :], sa[:, None], so)
    near = 0
    for m in range(M):
        for n in range(N):
            x = Fraction(int(acc[m, n])) * Fraction(float(ws[n])) * Fraction(float(sa[m])) \
                / Fraction(float(so))
            fl = x.numerator // x.denominator
            frac = x - fl
            exact = fl + (1 if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2) else 0)
            exact = max(-127, min(127, exact))
            if q[m, n] == exact:
                continue
            # only a near-tie may round the other way
            dist = abs(frac - Fraction(1, 2))
            assert dist <= abs(x) * Fraction(3, 2 ** 24) + Fraction(1, 2 ** 30), (m, n, float(x))
            assert abs(int(q[m, n]) - exact) == 1, (m, n)
            near += 1
    assert near <= 2                                  # near-ties are rare at these magnitudes
    # outputs spread over the whole code range, clipped at +-127 on both sides
    assert q.max() == 127 and q.min() == -127 and len(np.unique(q)) > 200


def test_w8a8_one_hot_and_bruteforce():
    rng = np.random.default_rng(42)
    N, K = 5, 32
    qw = rng.integers(-127, 128, (N, K)).astype(np.int8)
    qa = np.zeros((K, K), np.int8)
    qa[np.arange(K), np.arange(K)] = 1
    acc = O.int_accumulate(qa, qw)
    assert np.array_equal(acc, qw.T.astype(np.int64))           # "nt": row k picks column k
    qa = rng.integers(-127, 128, (3, K)).astype(np.int8)
    ws = rng.uniform(0.001, 0.01, N).astype(np.float32)
    sa = rng.uniform(0.01, 0.1, 3).astype(np.float32)
    so = np.float32(0.02)
    q = O.w8a8_gemm(qa, sa, qw, ws, out=O.OUT_I8, out_scale=so)
    for m in range(3):
        for n in range(N):
            a = sum(int(qa[m, k]) * int(qw[n, k]) for k in range(K))
            v = np.float32(np.float32(np.float32(a) * ws[n]) * sa[m])
            want = int(np.clip(np.rint(np.float32(v / so)), -127, 127))
            assert q[m, n] == want, (m, n)


# ---------------------------------------------------------------------------
# FP8 E4M3 x FP8 E4M3 (reading 11: the OCP E4M3 format)
# ---------------------------------------------------------------------------
def _e4m3_by_hand(c):
    """One code's value written out from the bit fields with math.ldexp."""
    s = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 0xF, c & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * math.ldexp(m, -9)
    return s * math.ldexp(8 + m, e - 10)


def test_e4m3_decode_closed_forms_and_table():
    vals = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c, v in [(0x7E, 448.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
                 (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x77, 240.0), (0xB8, -1.0),
                 (0xFE, -448.0), (0x00, 0.0)]:
        assert vals[c] == v, hex(c)
    assert np.signbit(vals[0x80]) and vals[0x80] == 0.0
    nan = np.isnan(vals)
    assert np.flatnonzero(nan).tolist() == [0x7F, 0xFF]       # the only NaNs
    for c in range(256):
        h = _e4m3_by_hand(c)
        assert (np.isnan(h) and np.isnan(vals[c])) or h == vals[c], hex(c)
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)                           # strictly increasing codes
    # each binade [2^e, 2^(e+1)) holds 8 values 2^(e-3) apart; the top one
    # holds 7, its last slot being the NaN
    for e in range(-6, 9):
        b = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        assert len(b) == (7 if e == 8 else 8) and np.all(np.diff(b) == 2.0 ** (e - 3)), e


def test_e4m3_encode_ties_saturation_and_library():
    c = np.arange(256, dtype=np.uint8)
    fin = ~np.isnan(O.e4m3_decode(c))
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(c[fin]).astype(np.float32)), c[fin])
    f32 = np.float32
    cases = [(1.0625, 0x38), (1.1875, 0x3A),                  # midpoints go to the even code
             (np.nextafter(f32(1.0625), f32(2)), 0x39), (np.nextafter(f32(1.0625), f32(0)), 0x38),
             (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),     # subnormal ties
             (460.0, 0x7E), (470.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE),   # saturation, no NaN
             (-0.0, 0x80), (-(2.0 ** -12), 0x80), (0.0, 0x00)]
    for x, want in cases:
        assert O.e4m3_encode(np.array([x], f32))[0] == want, (x, hex(want))
    # against the library conversion (round to nearest even, in range)
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(51)
    x = np.concatenate([rng.normal(0, 30, 20000), rng.normal(0, 0.01, 5000),
                        (O.e4m3_decode(c[:0x7E]) + O.e4m3_decode(c[1:0x7F])) / 2]).astype(f32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), ref)


def test_quantize_f8_rows():
    rng = np.random.default_rng(52)
    W = rng.normal(0, 0.02, (6, 256)).astype(np.float32)
    W[2] = 0
    q, s = O.quantize_f8(W)
    assert s[2] == 0 and not q[2].any()
    live = [0, 1, 3, 4, 5]
    assert np.array_equal(s[live], (np.max(np.abs(W[live]), axis=1) / np.float32(448)).astype(np.float32))
    i = np.argmax(np.abs(W[live]), axis=1)
    assert np.all(np.abs(O.e4m3_decode(q[live, i])) == 448.0)   # the row max is the top code
    rec = O.e4m3_decode(q[live]) * s[live, None]
    err = np.abs(W[live] - rec)
    # half a unit in the last of 3 mantissa bits, or half the subnormal step
    bound = np.maximum(np.abs(W[live]) * 2.0 ** -4, s[live, None] * 2.0 ** -10) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)
    # fp16 activations widen exactly
    A = rng.normal(0, 1, (3, 64)).astype(np.float16)
    qa, sa = O.quantize_f8(A)
    qb, sb = O.quantize_f8(A.astype(np.float32))
    assert np.array_equal(qa, qb) and np.array_equal(sa, sb)


def test_f8f8_one_hot_and_bruteforce():
    rng = np.random.default_rng(53)
    N, K = 4, 32
    qw = rng.integers(0, 256, (N, K)).astype(np.uint8)
    qw[(qw & 0x7F) == 0x7F] = 0x38                            # no NaN codes
    one = np.zeros((K, K), np.uint8)
    one[np.arange(K), np.arange(K)] = 0x38                    # 1.0 on the diagonal
    C = O.f8f8_gemm(one, np.ones(K, np.float32), qw, np.ones(N, np.float32), out=O.OUT_F32)
    assert np.array_equal(C, O.e4m3_decode(qw).T.astype(np.float32))   # "nt": row k picks column k
    qa = rng.integers(0, 256, (3, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0xB8
    sw = rng.uniform(0.001, 0.01, N).astype(np.float32)
    sa = rng.uniform(0.01, 0.1, 3).astype(np.float32)
    bias = rng.normal(0, 0.01, N).astype(np.float16)
    C = O.f8f8_gemm(qa, sa, qw, sw, bias=bias, out=O.OUT_F16)
    for m in range(3):
        for n in range(N):
            acc = math.fsum(_e4m3_by_hand(int(qa[m, k])) * _e4m3_by_hand(int(qw[n, k]))
                            for k in range(K))
            want = np.float16(acc * float(sw[n]) * float(sa[m]) + float(bias[n]))
            assert C[m, n] == want, (m, n)
    rows, cols = np.array([0, 2, 1]), np.array([3, 0, 1])
    e = O.f8f8_entries(qa, sa, qw, sw, rows, cols, bias=bias)
    assert np.array_equal(e, C[rows, cols])
