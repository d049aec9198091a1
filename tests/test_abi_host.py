"""Host-only checks of the C ABI: the library loads, exports every function
the header declares, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

import gemv_nibble_unpack_amd as G
from gemv_nibble_unpack_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "gemv_nibble_unpack.h")

# fake, 256-aligned device addresses: validation must fail before any use
P = ctypes.c_void_p(0x7F0000000000)
P2 = ctypes.c_void_p(0x7F0000100000)
MIS = ctypes.c_void_p(0x7F0000000002)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_header_and_library_agree():
    lib = G.load()
    names = declared_functions()
    assert len(names) == 34, names
    assert set(names) == set(L.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_constants_match_header():
    text = open(HEADER).read()
    for name in ["W4_OK", "W4_ERR_NULL", "W4_ERR_SHAPE", "W4_ERR_ALIGN", "W4_ERR_ARG",
                 "W4_ERR_WORKSPACE", "W4_ERR_HIP", "W4_ERR_SCRATCH", "W4_SYM_PER_CHANNEL", "W4_ASYM_GROUP",
                 "W4_OUT_F16", "W4_OUT_F32", "W4_OUT_I32", "W4_OUT_I8", "W4_IN_F16", "W4_IN_F32",
                 "W4_LAYOUT_W4A8", "W4_LAYOUT_W4A16", "W4_LAYOUT_W2A8", "W4_LAYOUT_W8A8",
                 "W4_OP_W4A8", "W4_OP_W4A16", "W4_OP_W2A8", "W4_OP_W2A16", "W4_OP_W8A8",
                 "W4_OP_F8F8",
                 "W4_GROUP_SIZE",
                 "W4_MAX_K"]:
        m = re.search(rf"#define\s+{name}\s+(-?\d+)", text)
        assert m, name
        assert int(m.group(1)) == getattr(L, name), name


def test_status_strings():
    lib = G.load()
    for s in range(-7, 1):
        assert lib.w4_status_string(s) != b"unknown status"
    assert lib.w4_status_string(-99) == b"unknown status"


def test_sizes():
    lib = G.load()
    # 4096x4096 W4A16: codes + fp16 scales + uint8 zeros, in whole tiles
    assert lib.prepack_bytes(L.W4_LAYOUT_W4A16, 4096, 4096) == 4096 * 2048 + 4096 * 32 * 3
    assert lib.prepack_bytes(L.W4_LAYOUT_W4A8, 11008, 4096) == 11008 * 2048
    # ragged shapes round up to 16 rows x 128 k (4-bit) or 256 k (2-bit) tiles
    assert lib.prepack_bytes(L.W4_LAYOUT_W4A8, 50, 208) == 4 * 2 * 1024
    assert lib.prepack_bytes(L.W4_LAYOUT_W2A8, 3200, 8640) == 200 * 34 * 1024
    assert lib.prepack_bytes(L.W4_LAYOUT_W4A16, 16, 100) == 0       # K % 128
    assert lib.prepack_bytes(7, 16, 128) == 0
    # INT8 weights: 16 rows x 64 k per 1 KiB tile
    assert lib.prepack_bytes(L.W4_LAYOUT_W8A8, 4096, 4096) == 4096 * 4096
    assert lib.prepack_bytes(L.W4_LAYOUT_W8A8, 50, 208) == 4 * 4 * 1024
    assert lib.w4_workspace_bytes(L.W4_LAYOUT_W4A16, 1, 4096, 4096) == 0
    assert lib.w4_workspace_bytes(L.W4_LAYOUT_W2A8, 1, 16, 131056) > 0
    # fused activation quantization: decode rows that fit LDS need nothing;
    # 16 rows of 4096 quantize into the workspace first (int8 rows + scales)
    assert lib.w4_fused_act_workspace_bytes(L.W4_LAYOUT_W4A8, 1, 4096, 4096) == 0
    # two launches: the 16 KiB counter area, then the int8 rows and their scales
    assert lib.w4_fused_act_workspace_bytes(L.W4_LAYOUT_W4A8, 16, 4096, 4096) == (
        16384 + 16 * 4096 + 256)
    assert lib.w4_fused_act_workspace_bytes(L.W4_LAYOUT_W4A16, 1, 4096, 4096) == 0


def test_error_paths_before_launch():
    lib = G.load()
    s = None
    # quantize_pack_w4
    assert lib.quantize_pack_w4(None, 4, 8, 0, -1, P, P2, None, s) == L.W4_ERR_NULL
    assert lib.quantize_pack_w4(P, 4, 7, 0, -1, P, P2, None, s) == L.W4_ERR_SHAPE
    assert lib.quantize_pack_w4(P, 4, 8, 5, -1, P, P2, None, s) == L.W4_ERR_ARG
    assert lib.quantize_pack_w4(P, 4, 8, 0, 128, P, P2, None, s) == L.W4_ERR_ARG
    assert lib.quantize_pack_w4(P, 4, 200, 1, 128, P, P2, P2, s) == L.W4_ERR_SHAPE
    assert lib.quantize_pack_w4(MIS, 4, 8, 0, -1, P, P2, None, s) == L.W4_ERR_ALIGN
    assert lib.quantize_pack_w4(P, 4, 256, 1, 128, P, P2, None, s) == L.W4_ERR_NULL
    # quantize_pack_w2 / ternary scale / quantize_a8
    assert lib.quantize_pack_w2(P, 4, 6, P2, s) == L.W4_ERR_SHAPE
    assert lib.ternary_scale_f16(P, 0, P2, s) == L.W4_ERR_SHAPE
    assert lib.quantize_a8(P, 3, 2, 16, P, P2, None, s) == L.W4_ERR_ARG
    assert lib.quantize_a8(P, 0, 2, 12, P, P2, None, s) == L.W4_ERR_SHAPE
    # prepack
    assert lib.prepack_w(0, P, None, None, 16, 24, P2, s) == L.W4_ERR_SHAPE
    assert lib.prepack_w(1, P, None, None, 16, 128, P2, s) == L.W4_ERR_NULL
    # matmuls
    args = (P, P, P, P, None, P2, L.W4_OUT_F16)
    assert lib.w4a8_gemm(*args, 1, 16, 24, None, 0, s) == L.W4_ERR_SHAPE
    assert lib.w4a8_gemm(*args, 1, 16, L.W4_MAX_K + 16, None, 0, s) == L.W4_ERR_SHAPE
    assert lib.w4a8_gemm(*args, 1, 0, 32, None, 0, s) == L.W4_ERR_SHAPE
    assert lib.w4a8_gemm(P, P, P, P, None, P2, 9, 1, 16, 32, None, 0, s) == L.W4_ERR_ARG
    assert lib.w4a8_gemm(None, P, P, P, None, P2, 0, 1, 16, 32, None, 0, s) == L.W4_ERR_NULL
    assert lib.w4a8_gemm(MIS, P, P, P, None, P2, 0, 1, 16, 32, None, 0, s) == L.W4_ERR_ALIGN
    assert lib.w4a8_gemm(None, None, None, None, None, None, 0, 0, 16, 32, None, 0, s) == L.W4_OK
    assert lib.w2a8_gemm(P, P, P, P, None, P2, 0, 1, 16, 131056, None, 0, s) == L.W4_ERR_WORKSPACE
    assert lib.w4a16_gemm(P, P, 64, None, P2, 1, 16, 128, None, 0, s) == L.W4_ERR_ARG
    assert lib.w4a16_gemm(P, P, 128, None, P2, 1, 16, 192, None, 0, s) == L.W4_ERR_SHAPE
    assert lib.w2a16_gemm(P, P, P, None, P2, 1, 16, 24, None, 0, s) == L.W4_ERR_SHAPE
    assert lib.w2a16_gemm(P, P, None, None, P2, 1, 16, 32, None, 0, s) == L.W4_ERR_NULL
    assert lib.w2a16_gemm(MIS, P, P, None, P2, 1, 16, 32, None, 0, s) == L.W4_ERR_ALIGN
    assert lib.w2a16_gemm(None, None, None, None, None, 0, 16, 32, None, 0, s) == L.W4_OK
    assert lib.w2a16_gemm(P, P, P, None, P2, 1, 16, 131056, None, 0, s) == L.W4_ERR_WORKSPACE
    # INT8 weights and the INT8-output matmul
    assert lib.quantize_pack_w8(P, 4, 24, P, P2, s) == L.W4_ERR_SHAPE
    assert lib.quantize_pack_w8(None, 4, 32, P, P2, s) == L.W4_ERR_NULL
    assert lib.quantize_pack_w8(P, 4, 32, MIS, P2, s) == L.W4_ERR_ALIGN
    a8 = (P, P, P, P)
    assert lib.w8a8_gemm(*a8, P2, P, P2, L.W4_OUT_I8, 1, 16, 32, None, 0, s) == L.W4_ERR_ARG
    assert lib.w8a8_gemm(*a8, None, None, P2, L.W4_OUT_I8, 1, 16, 32, None, 0, s) == L.W4_ERR_NULL
    assert lib.w8a8_gemm(*a8, None, P, P2, 7, 1, 16, 32, None, 0, s) == L.W4_ERR_ARG
    assert lib.w8a8_gemm(*a8, None, P, P2, L.W4_OUT_I8, 1, 16, 24, None, 0, s) == L.W4_ERR_SHAPE
    assert lib.w8a8_gemm(None, None, None, None, None, None, None, 0, 0, 16, 32, None, 0,
                         s) == L.W4_OK
    # FP8: per-row quantizer and the FP8 x FP8 matmul
    assert lib.quantize_f8(P, 2, 4, 32, P, P2, s) == L.W4_ERR_ARG
    assert lib.quantize_f8(P, 0, 4, 24, P, P2, s) == L.W4_ERR_SHAPE
    assert lib.quantize_f8(P, 0, 0, 32, P, P2, s) == L.W4_ERR_SHAPE
    assert lib.quantize_f8(None, 0, 4, 32, P, P2, s) == L.W4_ERR_NULL
    assert lib.quantize_f8(MIS, 0, 4, 32, P, P2, s) == L.W4_ERR_ALIGN
    f8 = (P, P, P, P, None, P2)
    assert lib.f8f8_gemm(*f8, L.W4_OUT_I32, 1, 16, 32, None, 0, s) == L.W4_ERR_ARG
    assert lib.f8f8_gemm(*f8, L.W4_OUT_F16, 1, 16, 24, None, 0, s) == L.W4_ERR_SHAPE
    assert lib.f8f8_gemm(None, P, P, P, None, P2, L.W4_OUT_F16, 1, 16, 32, None, 0,
                         s) == L.W4_ERR_NULL
    assert lib.f8f8_gemm(MIS, P, P, P, None, P2, L.W4_OUT_F16, 1, 16, 32, None, 0,
                         s) == L.W4_ERR_ALIGN
    assert lib.f8f8_gemm(None, None, None, None, None, None, 0, 0, 16, 32, None, 0, s) == L.W4_OK
    assert lib.f8f8_gemm(*f8, L.W4_OUT_F16, 1, 16, 131056, None, 0, s) == L.W4_ERR_WORKSPACE
    assert lib.w4_plan_workspace_bytes(L.W4_OP_F8F8, 1, 16, 131056) > 16384
    # the other A8 matmuls have no INT8 output
    assert lib.w4a8_gemm(P, P, P, P, None, P2, L.W4_OUT_I8, 1, 16, 32, None, 0, s) == L.W4_ERR_ARG
    # fused activation quantization
    for fn in (lib.w4a8_gemm_fused_act, lib.w2a8_gemm_fused_act):
        assert fn(P, 2, P, P, None, P2, 0, 1, 16, 32, None, 0, s) == L.W4_ERR_ARG
        assert fn(P, 0, P, P, None, P2, 9, 1, 16, 32, None, 0, s) == L.W4_ERR_ARG
        assert fn(P, 0, P, P, None, P2, 0, 1, 16, 24, None, 0, s) == L.W4_ERR_SHAPE
        assert fn(None, 0, P, P, None, P2, 0, 1, 16, 32, None, 0, s) == L.W4_ERR_NULL
        assert fn(MIS, 0, P, P, None, P2, 0, 1, 16, 32, None, 0, s) == L.W4_ERR_ALIGN
        assert fn(None, 0, None, None, None, None, 0, 0, 16, 32, None, 0, s) == L.W4_OK
        assert fn(P, 1, P, P, None, P2, 0, 16, 16, 131056, None, 0, s) == L.W4_ERR_WORKSPACE


def _names(lib, op, M, N, K):
    out = []
    buf = ctypes.create_string_buffer(64)
    for i in range(lib.w4_plan_count(op, M, N, K)):
        assert lib.w4_plan_name(op, M, N, K, i, buf, 64) == L.W4_OK
        out.append(buf.value.decode())
    return out


def test_noalloc_fused_entry_rejects_before_any_gpu_work():
    lib = G.load()
    text = open(HEADER).read()
    m = re.search(r"#define\s+W4_NOALLOC_SCRATCH_BYTES\s+\((\d+) \* 1024 \* 1024\)", text)
    assert m and int(m.group(1)) * 1024 * 1024 == L.W4_NOALLOC_SCRATCH_BYTES
    s = None
    f = lib.w4a8_gemm_fused_act_noalloc
    assert f(P, 0, P, P, None, P2, 0, 1, 16, 24, s) == L.W4_ERR_SHAPE
    assert f(P, 7, P, P, None, P2, 0, 1, 16, 32, s) == L.W4_ERR_ARG
    assert f(None, 0, P, P, None, P2, 0, 1, 16, 32, s) == L.W4_ERR_NULL
    assert f(MIS, 0, P, P, None, P2, 0, 1, 16, 32, s) == L.W4_ERR_ALIGN
    assert f(None, 0, None, None, None, None, 0, 0, 16, 32, s) == L.W4_OK
    # a shape whose scratch exceeds the static array: the int8 rows of a
    # two-launch call alone take M * K bytes
    M, K = 4096, 16384
    assert lib.w4_fused_act_workspace_bytes(L.W4_LAYOUT_W4A8, M, 4096, K) > \
        L.W4_NOALLOC_SCRATCH_BYTES
    assert f(P, 0, P, P, None, P2, 0, M, 4096, K, s) == L.W4_ERR_SCRATCH
    assert b"static" in lib.w4_status_string(L.W4_ERR_SCRATCH)


def test_read_probe_error_paths():
    lib = G.load()
    s = None
    sink = P2
    assert lib.w4_read_probe(None, 1024, 4, sink, s) == L.W4_ERR_NULL
    assert lib.w4_read_probe(P, 1024, 4, None, s) == L.W4_ERR_NULL
    assert lib.w4_read_probe(P, 0, 4, sink, s) == L.W4_ERR_SHAPE
    assert lib.w4_read_probe(P, 1000, 4, sink, s) == L.W4_ERR_SHAPE
    assert lib.w4_read_probe(P, 1024, 3, sink, s) == L.W4_ERR_ARG
    assert lib.w4_read_probe(MIS, 1024, 4, sink, s) == L.W4_ERR_ALIGN


def test_plan_table_candidates():
    lib = G.load()
    # decode shape: the decode kernel (8, 4 and 16 waves per block) and the
    # skinny kernel at each k split up to 1024 blocks (256 decode blocks, 32
    # skinny blocks unsplit; a skinny split keeps at least 2 of the 32 k tiles)
    assert _names(lib, L.W4_OP_W4A8, 1, 4096, 4096) == [
        "decode:ksplit=1", "decode:ksplit=1,waves=4", "decode:ksplit=1,waves=16",
        "decode:ksplit=2", "decode:ksplit=2,waves=4", "decode:ksplit=2,waves=16",
        "decode:ksplit=4", "decode:ksplit=4,waves=4", "decode:ksplit=4,waves=16", "skinny",
        "skinny:ksplit=2", "skinny:ksplit=4", "skinny:ksplit=8", "skinny:ksplit=16"]
    # 16 waves need per-wave staging and at most 8 tiles per wave, or no
    # staging and at most 4: not at 86 k tiles of 4 rows unsplit (rows too
    # long to stage, 6 tiles per wave)
    assert "decode:ksplit=1,waves=16" not in _names(lib, L.W4_OP_W4A16, 4, 4096, 11008)
    # built-in: 16 waves for long rows over 64..256 unsplit blocks only
    for op, M, N, K, want in ((L.W4_OP_W4A16, 1, 4096, 11008, "decode:ksplit=1,waves=16"),
                              (L.W4_OP_W2A8, 1, 3200, 8640, "decode:ksplit=1,waves=16"),
                              (L.W4_OP_W4A16, 1, 4096, 4096, "decode:ksplit=1"),
                              (L.W4_OP_W4A16, 1, 11008, 4096, "decode:ksplit=1"),
                              (L.W4_OP_W2A8, 1, 8640, 3200, "decode:ksplit=1,waves=4"),
                              (L.W4_OP_W4A8, 1, 11008, 4096, "decode:ksplit=1"),
                              # 4 rows of K=11008: the smallest split that
                              # lets each wave stage its own range
                              (L.W4_OP_W4A16, 4, 4096, 11008, "decode:ksplit=4"),
                              # one long row: 16 waves where 8 would need 16
                              # tiles each; a row the block can stage, unsplit
                              (L.W4_OP_W4A16, 1, 16384, 16384, "decode:ksplit=1,waves=16"),
                              (L.W4_OP_W4A16, 1, 28672, 8192, "decode:ksplit=1"),
                              (L.W4_OP_W4A16, 1, 8192, 28672, "decode:ksplit=1"),
                              # 4..16 rows of K <= 4096: 16 waves, staged per
                              # wave (4 rows) or not staged (16 rows)
                              (L.W4_OP_W4A16, 4, 4096, 4096, "decode:ksplit=1,waves=16"),
                              (L.W4_OP_W4A16, 16, 4096, 4096, "decode:ksplit=1,waves=16")):
        names = _names(lib, op, M, N, K)
        assert names[lib.w4_plan_current(op, M, N, K)] == want, (op, M, N, K)
    # prefill shape: plus the three GEMM block shapes of the INT4 x INT8 kernel
    assert _names(lib, L.W4_OP_W4A8, 2048, 4096, 4096) == [
        "decode:ksplit=1", "decode:ksplit=1,waves=16", "skinny", "skinny:rows=32",
        "skinny:rows=48", "skinny:rows=64", "gemm:128x256", "gemm:128x352", "gemm:256x352"]
    # above 16 rows the skinny kernel also runs with two to four row tiles per
    # block (three the built-in choice once one-tile blocks exceed the 512
    # resident and three-tile blocks fit one per CU, else two)
    names = _names(lib, L.W4_OP_W2A8, 128, 8640, 3200)
    assert [n for n in names if n.startswith("skinny") and "ksplit" not in n] == [
        "skinny", "skinny:rows=32", "skinny:rows=48", "skinny:rows=64"]
    assert names[lib.w4_plan_current(L.W4_OP_W2A8, 128, 8640, 3200)] == "skinny:rows=48"
    names = _names(lib, L.W4_OP_W2A16, 128, 8640, 3200)
    assert names[lib.w4_plan_current(L.W4_OP_W2A16, 128, 8640, 3200)] == "skinny:rows=48"
    # fp16 x 2-bit rows over 34 k tiles: two row tiles per block, split 7 ways
    names = _names(lib, L.W4_OP_W2A16, 128, 3200, 8640)
    assert names[lib.w4_plan_current(L.W4_OP_W2A16, 128, 3200, 8640)] == "skinny:rows=32,ksplit=7"
    # 40 rows: three row tiles at most
    assert not any("rows=64" in n for n in _names(lib, L.W4_OP_W2A16, 40, 1000, 2048))
    # 2048 rows x 16 column groups: 128 x 16 one-tile blocks exceed 512,
    # three-tile blocks (43 x 16) do not fit one per CU either: two tiles
    names = _names(lib, L.W4_OP_W2A16, 2048, 2048, 2048)
    assert names[lib.w4_plan_current(L.W4_OP_W2A16, 2048, 2048, 2048)] == "skinny:rows=32"
    names = _names(lib, L.W4_OP_W2A8, 128, 3200, 3200)
    assert names[lib.w4_plan_current(L.W4_OP_W2A8, 128, 3200, 3200)] == "skinny"
    # ternary weights above 16 rows: the 128 x 128 GEMM blocks, whole K and at
    # each distinct k split up to 1024 blocks (25 tiles, 34 k tiles)
    assert [n for n in _names(lib, L.W4_OP_W2A8, 128, 3200, 8640) if n.startswith("gemm")] == [
        "gemm:128x128"] + [f"gemm:128x128,ksplit={s}" for s in (2, 4, 7, 12, 17)]
    # splits are planned for blocks of up to 8 weight tiles only: the INT4
    # GEMM shapes always run over the whole K
    names = _names(lib, L.W4_OP_W4A8, 1100, 4004, 512)
    assert names[lib.w4_plan_current(L.W4_OP_W4A8, 1100, 4004, 512)] == "gemm:128x256"
    assert lib.w4_plan_workspace_bytes(L.W4_OP_W4A8, 1100, 4004, 512) == 0
    names = _names(lib, L.W4_OP_W2A8, 1100, 2000, 1024)
    assert names[lib.w4_plan_current(L.W4_OP_W2A8, 1100, 2000, 1024)] == "gemm:128x128,ksplit=2"
    # 2-bit fp16-activation products have no GEMM candidate; FP8 takes the
    # 128 x 128 block over the whole K (float32 sums are never split), INT8
    # weights the 128 x 128 block (built in once 128 blocks fill the chip
    # unsplit); W4A16 the fp16 GEMM's 128 x 256 or 128 x 352 block
    assert not any(n.startswith("gemm") for n in _names(lib, L.W4_OP_W2A16, 2048, 4096, 4096))
    names = _names(lib, L.W4_OP_F8F8, 2048, 4096, 4096)
    assert [n for n in names if n.startswith("gemm")] == ["gemm:128x128"]
    assert names[lib.w4_plan_current(L.W4_OP_F8F8, 2048, 4096, 4096)] == "gemm:128x128"
    assert lib.w4_plan_workspace_bytes(L.W4_OP_F8F8, 2048, 4096, 4096) == 0
    names = _names(lib, L.W4_OP_W4A16, 2048, 11008, 4096)
    assert [n for n in names if n.startswith("gemm")] == ["gemm:128x256", "gemm:128x352",
                                                          "gemm:128x384"]
    assert names[lib.w4_plan_current(L.W4_OP_W4A16, 2048, 11008, 4096)] == "gemm:128x384"
    assert names[lib.w4_plan_current(L.W4_OP_W4A16, 2048, 4096, 4096)] == "gemm:128x256"
    assert lib.w4_plan_workspace_bytes(L.W4_OP_W4A16, 2048, 11008, 4096) == 0
    names = _names(lib, L.W4_OP_W4A16, 128, 11008, 4096)
    assert not names[lib.w4_plan_current(L.W4_OP_W4A16, 128, 11008, 4096)].startswith("gemm")
    names = _names(lib, L.W4_OP_W8A8, 2048, 4096, 4096)
    assert names[lib.w4_plan_current(L.W4_OP_W8A8, 2048, 4096, 4096)] == "gemm:128x128"
    assert "gemm:128x128" in _names(lib, L.W4_OP_W8A8, 128, 4096, 4096)
    # a tiny-N, huge-K decode splits K 64 ways on its own (one output tile)
    names = _names(lib, L.W4_OP_W2A8, 1, 16, 131056)
    assert names[lib.w4_plan_current(L.W4_OP_W2A8, 1, 16, 131056)] == "decode:ksplit=64"


def test_plan_table_pin_and_workspace():
    lib = G.load()
    op, lay, M, N, K = L.W4_OP_W2A8, L.W4_LAYOUT_W2A8, 1, 16, 131056
    assert lib.w4_plan_reset() == L.W4_OK
    # built-in: 64-way split, 16 KiB counter area + 64 partial tiles of 1 KiB
    assert lib.w4_workspace_bytes(lay, M, N, K) == 16384 + 64 * 1024
    assert lib.w4_plan_pin(op, M, N, K, 0) == L.W4_OK          # decode, no split
    assert lib.w4_plan_current(op, M, N, K) == 0
    assert lib.w4_workspace_bytes(lay, M, N, K) == 0
    assert lib.w4_plan_workspace_bytes(op, M, N, K) == 0
    # the fp16-activation op on the same layout keeps its own (built-in) plan
    assert lib.w4_plan_workspace_bytes(L.W4_OP_W2A16, M, N, K) == 16384 + 64 * 1024
    # the pin is per (op, shape): another op or size keeps its built-in plan
    names = _names(lib, op, M, N, K - 256)
    assert names[lib.w4_plan_current(op, M, N, K - 256)] == "decode:ksplit=64"
    assert lib.w4_workspace_bytes(lay, M, N, K - 256) > 0
    # the fused entry points share the W2A8 op's plan: unsplit, the 128 KiB
    # row does not fit the LDS staging, so it is quantized into the workspace
    assert lib.w4_fused_act_workspace_bytes(lay, M, N, K) == 16384 + (K + 255) // 256 * 256 + 256
    builtin = _names(lib, op, M, N, K).index("decode:ksplit=64")
    assert lib.w4_plan_pin(op, M, N, K, -1) == L.W4_OK
    assert lib.w4_plan_current(op, M, N, K) == builtin
    assert lib.w4_plan_pin(op, M, N, K, 2) == L.W4_OK
    assert lib.w4_plan_pin(L.W4_OP_W4A8, 2048, 4096, 4096, 1) == L.W4_OK
    assert lib.w4_plan_current(L.W4_OP_W4A8, 2048, 4096, 4096) == 1
    assert lib.w4_plan_reset() == L.W4_OK
    assert lib.w4_plan_current(op, M, N, K) == builtin
    assert lib.w4_plan_current(L.W4_OP_W4A8, 2048, 4096, 4096) != 1


def test_plan_table_errors():
    lib = G.load()
    buf = ctypes.create_string_buffer(64)
    assert lib.w4_plan_count(6, 1, 16, 128) == L.W4_ERR_ARG
    assert lib.w4_plan_count(L.W4_OP_F8F8, 1, 16, 128) >= 2
    assert lib.w4_plan_count(-1, 1, 16, 128) == L.W4_ERR_ARG
    assert lib.w4_plan_count(L.W4_OP_W4A8, 0, 16, 128) == L.W4_ERR_SHAPE
    assert lib.w4_plan_count(L.W4_OP_W4A8, 1, 16, 24) == L.W4_ERR_SHAPE
    assert lib.w4_plan_count(L.W4_OP_W4A16, 1, 16, 192) == L.W4_ERR_SHAPE
    n = lib.w4_plan_count(L.W4_OP_W4A8, 1, 16, 128)
    assert n >= 2
    assert lib.w4_plan_name(L.W4_OP_W4A8, 1, 16, 128, n, buf, 64) == L.W4_ERR_ARG
    assert lib.w4_plan_name(L.W4_OP_W4A8, 1, 16, 128, 0, None, 64) == L.W4_ERR_NULL
    assert lib.w4_plan_name(L.W4_OP_W4A8, 1, 16, 128, 0, buf, 4) == L.W4_ERR_ARG
    assert lib.w4_plan_pin(L.W4_OP_W4A8, 1, 16, 128, n) == L.W4_ERR_ARG
    assert lib.w4_plan_pin(L.W4_OP_W4A8, 1, 16, 128, -2) == L.W4_ERR_ARG
    assert lib.w4_plan_pin(L.W4_OP_W4A8, 1, 16, 24, 0) == L.W4_ERR_SHAPE
    assert lib.w4_plan_workspace_bytes(9, 1, 16, 131056) == 0
    assert lib.w4_plan_workspace_bytes(L.W4_OP_W2A8, 0, 16, 131056) == 0


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        G.quantize_pack_w4(torch.zeros(4, 8))


def test_graph_entry_points_reject_null_before_any_hip_call():
    lib = G.load()
    assert lib.w4_graph_begin(None) == L.W4_ERR_NULL
    h = ctypes.c_void_p()
    assert lib.w4_graph_end(None, ctypes.byref(h)) == L.W4_ERR_NULL
    assert lib.w4_graph_end(P, None) == L.W4_ERR_NULL
    assert lib.w4_graph_update(None, P) == L.W4_ERR_NULL
    assert lib.w4_graph_update(P, None) == L.W4_ERR_NULL
    assert lib.w4_graph_launch(None, None) == L.W4_ERR_NULL
    assert lib.w4_graph_kernel_nodes(None) == L.W4_ERR_NULL
    assert lib.w4_graph_destroy(None) == L.W4_OK


def test_step_graph_needs_a_stream_of_its_own():
    class Default:
        cuda_stream = 0
    with pytest.raises(ValueError):
        G.StepGraph(Default())
    with pytest.raises(ValueError):
        G.StepGraph(None)
