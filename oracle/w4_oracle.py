"""CPU oracle for the INT4 / ternary-INT2 weight matmul (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module. It shares no code with the HIP library and
imports nothing from it.

Sources (cited by page title and section):

* [INT4 page] "Accelerating LLM inference with CUDA Graph and INT4
  quantization" (基于CUDA Graph 和 INT4 量化加速大语言模型推理过程), Part 1:
  step 1 weight quantization (symmetric scale from the largest magnitude,
  round, clip, two 4-bit values per byte), step 2 activation quantization
  (dynamic scale, round), step 3 the INT4 GEMM dataflow (unpack, 8-bit dot
  products into INT32, multiply by the scales, optional bias), step 4
  dequantization (INT32 result times weight_scale * activation_scale).
* [BitBLAS page] "BitBLAS practical guide: mixed-precision matmul in vLLM"
  (BitBLAS实战指南：在vLLM中集成混合精度计算，降低70%内存使用): section
  "What is BitBLAS" (the problem statement C[M,N] = A[M,K] x W[N,K], layout
  "nt"), the data-type table (FP16 x INT4, FP16 x INT2, INT8 x INT2), the memory-saving
  list (INT4 saves 75 %, INT2 87.5 % against FP16), "Advanced features 2:
  weight group quantization" (group_size 128, with scaling, with zeros,
  zeros_mode "original"), and the BitNet-b1.58 case (ternary weights).

Readings taken where the pages are silent or contradict themselves (each is
listed again in the design notes):

1. INT4 symmetric range is [-7, 7] with scale = max|w| / 7. The INT4 page
   prints 127, which it itself calls the INT8 range; 127 is kept for the INT8
   activations only. Code -8 is never produced.
2. Scales are per output channel (one per row n of W) for the symmetric
   scheme; the page's formula takes the max over "the weight tensor".
3. round() is round-half-to-even; divisions are IEEE float32 divisions
   (the precision the kernels decide codes in).
4. Nibble order: element 2j of a row goes to the low nibble of byte j, 2j+1
   to the high nibble. Crumbs (2-bit) are little-endian within a byte.
   Signed values are stored as two's complement.
5. Group quantization (asymmetric uINT4, zeros_mode "original"): over each
   group of 128 consecutive k, s16 = fp16((max - min) / 15), every later
   step uses the fp16-rounded scale, z = clip(rint(-min / s), 0, 15),
   q = clip(rint(w / s) + z, 0, 15), and w is reconstructed as (q - z) * s.
   A group with s == 0 gets q = z = 0.
6. Accumulation for FP16 x INT4 (and FP16 x INT2) is float32 in the kernels
   (the BitBLAS example names fp16; fp16 accumulation over K = 11008 would
   not meet the output tolerance); the oracle accumulates in float64.
7. Activations are quantized per token (row m), dynamically, to [-127, 127].
8. Ternary codes are inputs; their per-tensor scale is fp16(mean |src|) of
   the float32 source, summed in float64.
9. FP16 x INT2 (a table row with no scheme on the pages) uses the ternary
   codes and tensor scale of reading 8, the only INT2 weights the pages
   describe: C = fp16(s * sum a * c + bias).
10. INT8 x INT8 with INT8 output: weights use the INT4 page's printed
    formula as it stands (scale = max|w| / 127 per row, codes in [-127,
    127]); the INT8 output is the INT32 result re-quantized for a following
    INT8 layer by a given per-tensor output scale: v = acc * w_scale *
    a_scale in float32, left to right, code = clip(rint(v / out_scale), -127,
    127) with a float32 division (the precision the kernel decides it in); an
    output scale of 0 gives 0. The INT8 output takes no bias.
11. FP8_E4M3 x FP8_E4M3 (the table's last row: FP32 accumulate, FP16
    output). The pages name the format only; E4M3 is taken as the OCP 8-bit
    floating-point format: 1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits, subnormals m * 2^-9 at exponent 0, no infinities, S.1111.111 the
    only NaN, largest magnitude 448. Conversion to E4M3 rounds to nearest,
    ties to the even code, keeps the sign of zero, and saturates at +-448.
    Both operands are quantized per row (activations per token, weights per
    output channel) the way the INT8 rows are: scale = max|x| / 448 in
    float32, code = E4M3(x / scale) with a float32 division; a zero row gets
    scale 0 and code 0. C = out(sum_k a_k * w_k * w_scale[n] * a_scale[m]
    + bias[n]), the sum of exact products taken in float64 here (float32 in
    the kernels).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "quantize_w4_sym",
    "quantize_w4_group",
    "pack_int4",
    "unpack_int4",
    "pack_int2",
    "unpack_int2",
    "ternary_scale",
    "quantize_a8",
    "int_accumulate",
    "int_accumulate_entries",
    "int_accumulate_f64",
    "dequant_epilogue",
    "w4a8_gemm",
    "w2a16_gemm",
    "quantize_w8_sym",
    "requantize_i8",
    "w8a8_gemm",
    "e4m3_decode",
    "e4m3_encode",
    "quantize_f8",
    "f8f8_gemm",
    "f8f8_entries",
    "E4M3_MAX",
    "OUT_I8",
    "w2a16_entries",
    "w2a8_gemm",
    "w4a16_gemm",
    "w4a16_entries",
    "OUT_F16",
    "OUT_F32",
    "OUT_I32",
]

OUT_F16, OUT_F32, OUT_I32, OUT_I8 = "f16", "f32", "i32", "i8"

_F32 = np.float32


# ----------------------------------------------------------------------------
# weight quantization
# ----------------------------------------------------------------------------
def quantize_w4_sym(W):
    """Symmetric per-output-channel INT4 codes and float32 scales.

    INT4 page, Part 1 step 1: scale = largest magnitude / Q, code =
    round(w / scale), clipped to the symmetric range; Q = 7 for INT4
    (reading 1). One scale per row n (reading 2). Returns (q int8 [N,K] in
    [-7,7], s float32 [N]).
    """
    W = np.ascontiguousarray(W, dtype=_F32)
    amax = np.max(np.abs(W), axis=1)              # exact in float32
    s = (amax / _F32(7.0)).astype(_F32)           # IEEE float32 division
    q = np.zeros(W.shape, dtype=np.int8)
    live = s > 0
    if np.any(live):
        r = np.rint(W[live] / s[live, None])       # float32 divide, half-even
        q[live] = np.clip(r, -7, 7).astype(np.int8)
    return q, s


def quantize_w4_group(W, group_size=128):
    """Asymmetric uINT4 codes with fp16 group scales and uint8 zeros.

    BitBLAS page, "Advanced features 2: weight group quantization"
    (group_size=128, with_scaling, with_zeros, zeros_mode "original"), with
    the min/max asymmetric scheme of reading 5. Returns (q uint8 [N,K] in
    [0,15], s float16 [N,K/g], z uint8 [N,K/g]).
    """
    W = np.ascontiguousarray(W, dtype=_F32)
    N, K = W.shape
    if K % group_size:
        raise ValueError("K must be a multiple of group_size")
    G = K // group_size
    Wg = W.reshape(N, G, group_size)
    mn = Wg.min(axis=2)
    mx = Wg.max(axis=2)
    s16 = ((mx - mn) / _F32(15.0)).astype(np.float16)   # fp32 op, then RNE to fp16
    sf = s16.astype(_F32)
    z = np.zeros((N, G), dtype=np.uint8)
    q = np.zeros((N, G, group_size), dtype=np.uint8)
    live = sf > 0
    if np.any(live):
        zl = np.clip(np.rint(-mn[live] / sf[live]), 0, 15)
        ql = np.clip(np.rint(Wg[live] / sf[live][:, None]) + zl[:, None], 0, 15)
        z[live] = zl.astype(np.uint8)
        q[live] = ql.astype(np.uint8)
    return q.reshape(N, K), s16, z


def ternary_scale(src):
    """Per-tensor fp16 scale of a ternary weight: fp16(mean |src|).

    BitBLAS page, BitNet-b1.58 case (ternary weights); the absmean scale is
    reading 8. The sum is taken in float64 over the float32 source.
    """
    src = np.asarray(src, dtype=_F32)
    mean = np.abs(src.astype(np.float64)).sum() / src.size
    return np.float16(mean)


# ----------------------------------------------------------------------------
# packing
# ----------------------------------------------------------------------------
def pack_int4(q):
    """Two 4-bit codes per byte: element 2j -> low nibble, 2j+1 -> high.

    INT4 page, Part 1 step 1 ("storage": two INT4 weights in one byte);
    nibble order is reading 4. Accepts signed [-8,7] or unsigned [0,15]
    codes; returns uint8 [N, K/2].
    """
    q = np.asarray(q)
    if q.shape[-1] % 2:
        raise ValueError("K must be even")
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(b, signed):
    """Inverse of pack_int4; signed=True gives two's-complement [-8,7]."""
    b = np.asarray(b, dtype=np.uint8)
    lo = (b & 0xF).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    if signed:
        lo = np.where(lo >= 8, lo - 16, lo)
        hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int16)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out.astype(np.int8 if signed else np.uint8)


def pack_int2(c):
    """Four 2-bit two's-complement codes per byte, element 4j+i at bits 2i.

    BitBLAS page data-type table (INT8 x INT2) and memory list (INT2 is one
    eighth of FP16); crumb order is reading 4.
    """
    c = np.asarray(c)
    if c.shape[-1] % 4:
        raise ValueError("K must be a multiple of 4")
    u = (c.astype(np.int16) & 0x3).astype(np.uint8)
    return (u[..., 0::4] | (u[..., 1::4] << 2) | (u[..., 2::4] << 4)
            | (u[..., 3::4] << 6)).astype(np.uint8)


def unpack_int2(b):
    """Inverse of pack_int2: 2-bit two's complement -> int8 in [-2, 1]."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (4 * b.shape[-1],), dtype=np.int16)
    for i in range(4):
        v = ((b >> (2 * i)) & 0x3).astype(np.int16)
        out[..., i::4] = np.where(v >= 2, v - 4, v)
    return out.astype(np.int8)


# ----------------------------------------------------------------------------
# activations
# ----------------------------------------------------------------------------
def quantize_a8(A):
    """Per-token dynamic INT8 activations.

    INT4 page, Part 1 step 2: quantized = round(activation / scale), with a
    dynamic scale; per token and symmetric [-127, 127] (reading 7), scale =
    max|a| / 127 in float32. fp16 inputs widen exactly to float32. Returns
    (qa int8 [M,K], sa float32 [M], rowsum int32 [M] = sum_k qa).
    """
    A32 = np.ascontiguousarray(A).astype(_F32)
    amax = np.max(np.abs(A32), axis=1) if A32.shape[1] else np.zeros(A32.shape[0], _F32)
    sa = (amax / _F32(127.0)).astype(_F32)
    qa = np.zeros(A32.shape, dtype=np.int8)
    live = sa > 0
    if np.any(live):
        r = np.rint(A32[live] / sa[live, None])
        qa[live] = np.clip(r, -127, 127).astype(np.int8)
    rowsum = qa.astype(np.int64).sum(axis=1).astype(np.int32)
    return qa, sa, rowsum


# ----------------------------------------------------------------------------
# matmul
# ----------------------------------------------------------------------------
def int_accumulate(qa, qw):
    """INT32 accumulators acc[m,n] = sum_k qa[m,k] * qw[n,k] ("nt").

    BitBLAS page "What is BitBLAS": C[M,N] = A[M,K] x W[N,K], both operands
    K-contiguous. INT4 page Part 1 step 3: 8-bit products summed into INT32.
    Computed exactly in int64 and checked to fit int32.
    """
    acc = np.asarray(qa, np.int64) @ np.asarray(qw, np.int64).T
    if acc.size and (acc.max() > 2**31 - 1 or acc.min() < -(2**31)):
        raise OverflowError("accumulator exceeds int32")
    return acc


def int_accumulate_f64(qa, qw):
    """The INT32 accumulators of ``int_accumulate`` through a float64 matrix
    product of the codes (a library routine, so full-size outputs check in
    seconds where the int64 product would take minutes).

    Exact: every product of two codes is an integer of magnitude at most
    max|qa| * max|qw|, and every partial sum, in whatever order the routine
    adds, is an integer no larger than K times that; below 2^53 float64
    represents all of them exactly, so no addition rounds. The bound is
    checked from the inputs before the product is taken.
    """
    qa = np.asarray(qa)
    qw = np.asarray(qw)
    K = qa.shape[1]
    amax = int(np.max(np.abs(qa.astype(np.int64)))) if qa.size else 0
    wmax = int(np.max(np.abs(qw.astype(np.int64)))) if qw.size else 0
    if K * amax * wmax >= 2**53:
        raise OverflowError("float64 sums would round")
    acc = (qa.astype(np.float64) @ qw.astype(np.float64).T).astype(np.int64)
    if acc.size and (acc.max() > 2**31 - 1 or acc.min() < -(2**31)):
        raise OverflowError("accumulator exceeds int32")
    return acc


def int_accumulate_entries(qa, qw, rows, cols):
    """The same sums for selected (rows[i], cols[i]) entries only."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    a = np.asarray(qa, np.int64)[rows]
    w = np.asarray(qw, np.int64)[cols]
    return np.einsum("ik,ik->i", a, w)


def dequant_epilogue(acc, ws, sa, bias, out):
    """Scale INT32 accumulators back to real numbers.

    INT4 page, Part 1 steps 3-4: multiply the INT32 result by
    weight_scale * activation_scale, optionally add a bias, convert to the
    output precision (or hand back the INT32 result). ``acc`` is [M,N] (or
    a flat vector of entries with matching ``ws``/``sa``/``bias``). The
    product is formed in float64 and rounded once to the output type.
    """
    acc = np.asarray(acc, np.int64)
    if out == OUT_I32:
        return acc.astype(np.int32)
    v = acc.astype(np.float64) * np.asarray(ws, np.float64) * np.asarray(sa, np.float64)
    if bias is not None:
        v = v + np.asarray(bias, np.float64)
    if out == OUT_F32:
        return v.astype(_F32)
    if out == OUT_F16:
        return v.astype(np.float16)
    raise ValueError(out)


def w4a8_gemm(qa, sa, qw, ws, bias=None, out=OUT_F16):
    """W4A8: INT8 activations x symmetric INT4 weights -> out.

    ``qa`` int8 [M,K], ``sa`` float32 [M], ``qw`` int8 codes [N,K] in
    [-7,7] (unpacked), ``ws`` float32 [N], ``bias`` fp16 [N] or None.
    """
    acc = int_accumulate(qa, qw)
    return dequant_epilogue(acc, np.asarray(ws, np.float32)[None, :],
                            np.asarray(sa, np.float32)[:, None],
                            None if bias is None else np.asarray(bias)[None, :], out)


def w2a8_gemm(qa, sa, codes, scale16, bias=None, out=OUT_F16):
    """W2A8: INT8 activations x ternary codes with one fp16 tensor scale."""
    acc = int_accumulate(qa, codes)
    ws = np.float64(np.float16(scale16))
    return dequant_epilogue(acc, ws, np.asarray(sa, np.float32)[:, None],
                            None if bias is None else np.asarray(bias)[None, :], out)


def w2a16_gemm(A16, codes, scale16, bias=None):
    """W2A16: fp16 activations x ternary codes with one fp16 tensor scale.

    BitBLAS page data-type table row FP16 x INT2, on the ternary weights of
    the BitNet-b1.58 case (reading 8). C[m,n] = fp16(s * sum_k a[m,k] *
    c[n,k] + bias[n]); the sum is taken in float64 (reading 6).
    """
    C = np.asarray(A16).astype(np.float64) @ np.asarray(codes).astype(np.float64).T
    C = C * np.float64(np.float16(scale16))
    if bias is not None:
        C = C + np.asarray(bias).astype(np.float64)[None, :]
    return C.astype(np.float16)


def w2a16_entries(A16, codes, scale16, rows, cols, bias=None):
    """The W2A16 result for selected (rows[i], cols[i]) entries only."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    a = np.asarray(A16)[rows].astype(np.float64)
    c = np.asarray(codes)[cols].astype(np.float64)
    v = np.einsum("ik,ik->i", a, c) * np.float64(np.float16(scale16))
    if bias is not None:
        v = v + np.asarray(bias).astype(np.float64)[cols]
    return v.astype(np.float16)


def quantize_w8_sym(W):
    """Symmetric per-output-channel INT8 codes and float32 scales.

    INT4 page, Part 1 step 1 exactly as printed: scale = largest magnitude /
    127, code = round(w / scale) clipped to [-127, 127] (reading 10), one
    scale per row n (reading 2), float32 division and half-even rounding
    (reading 3). Returns (q int8 [N,K], s float32 [N]).
    """
    W = np.ascontiguousarray(W, dtype=_F32)
    amax = np.max(np.abs(W), axis=1)
    s = (amax / _F32(127.0)).astype(_F32)
    q = np.zeros(W.shape, dtype=np.int8)
    live = s > 0
    if np.any(live):
        r = np.rint(W[live] / s[live, None])
        q[live] = np.clip(r, -127, 127).astype(np.int8)
    return q, s


def requantize_i8(acc, ws, sa, out_scale):
    """INT8 output codes from INT32 accumulators (reading 10).

    BitBLAS page data-type table row INT8 x INT8 -> INT8; INT4 page, Part 1
    step 3 (the INT32 result handed to a following quantized layer). ``acc``
    [M,N] (or flat entries with matching ``ws``/``sa``); the product and the
    division are taken in float32, in that order.
    """
    v = (np.asarray(acc, np.int64).astype(_F32) * np.asarray(ws, _F32)).astype(_F32)
    v = (v * np.asarray(sa, _F32)).astype(_F32)
    so = _F32(out_scale)
    if not so > 0:
        return np.zeros(v.shape, np.int8)
    return np.clip(np.rint(v / so), -127, 127).astype(np.int8)


def w8a8_gemm(qa, sa, qw, ws, bias=None, out=OUT_F16, out_scale=None):
    """W8A8: INT8 activations x INT8 weights, exact INT32 sums, then the
    dequantized (f16/f32), raw (i32) or re-quantized (i8) output."""
    acc = int_accumulate(qa, qw)
    if out == OUT_I8:
        return requantize_i8(acc, np.asarray(ws, _F32)[None, :], np.asarray(sa, _F32)[:, None],
                             out_scale)
    return dequant_epilogue(acc, np.asarray(ws, np.float64)[None, :],
                            np.asarray(sa, np.float32)[:, None],
                            None if bias is None else np.asarray(bias)[None, :], out)


def _dequant_group(q, s16, z, group_size):
    """(q - z) * s per element in float64 (zeros_mode "original")."""
    N, K = q.shape
    G = K // group_size
    d = (q.reshape(N, G, group_size).astype(np.float64)
         - z.astype(np.float64)[:, :, None]) * s16.astype(np.float64)[:, :, None]
    return d.reshape(N, K)


def w4a16_gemm(A16, q, s16, z, group_size=128, bias=None):
    """W4A16: fp16 activations x group-quantized uINT4 weights -> fp16.

    BitBLAS page data-type table row FP16 x INT4 and "Advanced features 2"
    (group scales and zeros). C[m,n] = fp16(sum_k a[m,k] * (q[n,k] - z) * s
    + bias[n]), with the sum in float64 (reading 6).
    """
    Wd = _dequant_group(np.asarray(q), np.asarray(s16), np.asarray(z), group_size)
    C = np.asarray(A16).astype(np.float64) @ Wd.T
    if bias is not None:
        C = C + np.asarray(bias).astype(np.float64)[None, :]
    return C.astype(np.float16)


def w4a16_entries(A16, q, s16, z, rows, cols, group_size=128, bias=None):
    """The W4A16 result for selected (rows[i], cols[i]) entries only."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    Wd = _dequant_group(np.asarray(q)[cols], np.asarray(s16)[cols],
                        np.asarray(z)[cols], group_size)
    a = np.asarray(A16)[rows].astype(np.float64)
    v = np.einsum("ik,ik->i", a, Wd)
    if bias is not None:
        v = v + np.asarray(bias).astype(np.float64)[cols]
    return v.astype(np.float16)


# ----------------------------------------------------------------------------
# FP8 E4M3 x FP8 E4M3 (reading 11)
# ----------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Values of E4M3 codes in float64, from the bit fields (reading 11):
    exponent 0 -> m * 2^-9; else (1 + m / 8) * 2^(e - 7); 0x7F / 0xFF NaN."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag


# the 127 non-negative finite values, in code order (increasing)
_E4M3_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x):
    """E4M3 codes (uint8) of float32 values: the nearest of the 127 finite
    magnitudes, ties to the even code, sign kept (also for zero), magnitudes
    above 448 saturated to 448 (reading 11). A plain nearest-neighbour search
    over the value table, not a bit-level conversion."""
    x = np.asarray(x, _F32)
    a = np.minimum(np.abs(x).astype(np.float64), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")      # first value >= a
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    code = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    code = np.where(tie, np.where(lo % 2 == 0, lo, hi), code)
    code = np.where(_E4M3_POS[hi] == a, hi, code)          # exact values
    neg = np.signbit(x)
    return (code.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)).astype(np.uint8)


def quantize_f8(X):
    """Per-row E4M3 quantization (reading 11): s = max|x| / 448 in float32,
    code = E4M3(fl32(x / s)); zero rows give s = 0 and code 0. X is float32
    (weights) or fp16 (activations, widened exactly). Returns (codes uint8
    [R,K], s float32 [R])."""
    X = np.asarray(X)
    X = X.astype(_F32) if X.dtype != _F32 else np.ascontiguousarray(X)
    amax = np.max(np.abs(X), axis=1)
    s = (amax / _F32(E4M3_MAX)).astype(_F32)
    q = np.zeros(X.shape, dtype=np.uint8)
    live = s > 0
    if np.any(live):
        q[live] = e4m3_encode((X[live] / s[live, None]).astype(_F32))
    return q, s


def _f8_out(v, bias, out):
    if bias is not None:
        v = v + bias
    return v.astype(np.float16) if out == OUT_F16 else v.astype(np.float32)


def f8f8_gemm(qa, sa, qw, sw, bias=None, out=OUT_F16):
    """FP8 x FP8: C[m,n] = out(sum_k dec(qa[m,k]) dec(qw[n,k]) * sw[n] * sa[m]
    + bias[n]); the products are exact and summed in float64."""
    acc = e4m3_decode(qa) @ e4m3_decode(qw).T
    v = acc * np.asarray(sw, np.float64)[None, :] * np.asarray(sa, np.float64)[:, None]
    b = None if bias is None else np.asarray(bias).astype(np.float64)[None, :]
    return _f8_out(v, b, out)


def f8f8_entries(qa, sa, qw, sw, rows, cols, bias=None, out=OUT_F16):
    """The FP8 x FP8 result for selected (rows[i], cols[i]) entries only."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    a = e4m3_decode(np.asarray(qa)[rows])
    w = e4m3_decode(np.asarray(qw)[cols])
    v = np.einsum("ik,ik->i", a, w) * np.asarray(sw, np.float64)[cols] * \
        np.asarray(sa, np.float64)[rows]
    b = None if bias is None else np.asarray(bias).astype(np.float64)[cols]
    return _f8_out(v, b, out)
