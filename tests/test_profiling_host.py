"""Host logic of the profiler summaries (no GPU): rocprofv3 CSV parsing, the
byte-counter calibration of the traffic record, the source-hash check that
retires a record once the kernels change, and the matrix-core summary."""
import csv
import json

import pytest

from gemv_nibble_unpack_amd import profiling as P

HDR = ["Correlation_Id", "Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name",
       "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _counters(d, rows):
    """rows: (kernel, counter, value) or (kernel, counter, value, grid threads)."""
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HDR)
        for i, row in enumerate(rows):
            kernel, counter, value = row[:3]
            grid = row[3] if len(row) > 3 else 1024
            w.writerow([i, i, grid, kernel, counter, value, 1000 * i, 1000 * i + 500])


def test_trace_summary(tmp_path):
    d = tmp_path / "t"
    d.mkdir()
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z",
                    "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"])
        for ns in (4000, 5000, 6000):
            w.writerow(["k_gemv", 131072, 1, 1, 512, 0, ns])
        w.writerow(["k_gemv", 352256, 1, 1, 512, 0, 7000])     # another shape, listed apart
        w.writerow(["copy", 512, 1, 1, 512, 0, 1000])
    out = tmp_path / "s.md"
    P.summarize_trace(str(d), str(out), "cmd")
    text = out.read_text()
    assert "`k_gemv` | 131072x1x1 / 512 | 3 | 5.00 | 5.00 | 4.00 |" in text
    assert "`k_gemv` | 352256x1x1 / 512 | 1 | 7.00 | 7.00 | 7.00 |" in text
    assert text.index("131072x1x1") < text.index("352256x1x1") < text.index("copy")  # by total
    assert "Command: `cmd`" in text


def test_traffic_calibration_and_hash(tmp_path, monkeypatch):
    # the copy kernel moves 2048 KiB; its counters read 1024 (fetch) and
    # 2048 (write) KiB, so a counter KiB is worth 2 KiB fetched, 1 KiB written
    _counters(tmp_path / "f", [("bitwise_not copy", "FETCH_SIZE", 1024.0),
                               ("k_gemv<1>", "FETCH_SIZE", 100.0),
                               ("k_gemv<1>", "FETCH_SIZE", 300.0)])
    _counters(tmp_path / "w", [("bitwise_not copy", "WRITE_SIZE", 2048.0),
                               ("k_gemv<1>", "WRITE_SIZE", 8.0)])
    out = tmp_path / "t.json"
    rec = P.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(out), "k_gemv",
                              2048 * 1024, "cmd")
    assert rec["read_bytes_per_launch"] == 200.0 * 2048     # median 200 KiB x 2
    assert rec["write_bytes_per_launch"] == 8.0 * 1024
    assert P.load_traffic(str(out))["traffic_bytes_per_launch"] == rec["traffic_bytes_per_launch"]
    # a record taken from other kernel sources is not used
    monkeypatch.setattr(P, "kernel_source_hash", lambda: "different")
    assert P.load_traffic(str(out)) is None
    assert P.load_traffic(str(tmp_path / "missing.json")) is None
    with pytest.raises(KeyError):
        P.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(out), "k_gemm",
                            2048 * 1024, "cmd")


def test_traffic_of_one_launch_shape(tmp_path):
    # two shapes of one kernel: the grid filter keeps one, and the copy
    _counters(tmp_path / "f", [("bitwise_not copy", "FETCH_SIZE", 1024.0, 65536),
                               ("k_gemv<1>", "FETCH_SIZE", 100.0, 131072),
                               ("k_gemv<1>", "FETCH_SIZE", 900.0, 352256)])
    _counters(tmp_path / "w", [("bitwise_not copy", "WRITE_SIZE", 2048.0, 65536),
                               ("k_gemv<1>", "WRITE_SIZE", 8.0, 131072),
                               ("k_gemv<1>", "WRITE_SIZE", 24.0, 352256)])
    out = tmp_path / "t.json"
    rec = P.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(out), "k_gemv",
                              2048 * 1024, "cmd", grid=352256)
    assert rec["read_bytes_per_launch"] == 900.0 * 2048
    assert rec["write_bytes_per_launch"] == 24.0 * 1024
    assert rec["grid_threads"] == 352256


def test_mfma_summary(tmp_path):
    _counters(tmp_path / "u", [("k_gemm<0>", "MfmaUtil", 49.0), ("k_gemm<0>", "MfmaUtil", 51.0),
                               ("k_quant_a8", "MfmaUtil", 0.0)])
    _counters(tmp_path / "r", [("k_gemm<0>", "SQ_INSTS_VALU_MFMA_MOPS_I8", 1024.0),
                               ("k_gemm<0>", "SQ_VALU_MFMA_BUSY_CYCLES", 256.0),
                               ("k_gemm<0>", "GRBM_GUI_ACTIVE", 4096.0)])
    out = tmp_path / "m.md"
    P.summarize_mfma(str(tmp_path / "u"), str(tmp_path / "r"), str(out), "k_gemm",
                     1024 * 512 / 2, ["c1", "c2"])
    text = out.read_text()
    assert "| 50.0 % |" in text                                  # median of the gemm launches
    assert "| 5.2429e+05 |" in text and "| 2.0000 |" in text     # executed = 2 x algorithmic
    assert "* `c1`" in text and "* `c2`" in text


def test_counter_summary(tmp_path):
    # two passes; medians per launch, per wave from SQ_WAVES, launch-size filter
    _counters(tmp_path / "a", [("k_skinny<2>", "SQ_WAVES", 1600.0, 102400),
                               ("k_skinny<2>", "SQ_WAVES", 1600.0, 102400),
                               ("k_skinny<2>", "SQ_INSTS_VALU", 1600.0 * 500, 102400),
                               ("k_skinny<2>", "SQ_INSTS_VALU", 1600.0 * 700, 102400),
                               ("k_skinny<2>", "SQ_INSTS_VALU", 9.0, 4096),      # other shape
                               ("other", "SQ_WAVES", 5.0, 102400)])
    _counters(tmp_path / "b", [("k_skinny<2>", "SQ_LDS_BANK_CONFLICT", 300.0, 102400),
                               ("k_skinny<2>", "SQ_ACTIVE_INST_LDS", 150.0, 102400)])
    out = tmp_path / "c.md"
    per = P.summarize_counters([str(tmp_path / "a"), str(tmp_path / "b")], str(out), "k_skinny",
                               ["cmd a", "cmd b"], grid=102400)
    assert per["SQ_INSTS_VALU"] == 1600.0 * 600
    text = out.read_text()
    assert "| SQ_INSTS_VALU | 960000 | 600.0 |" in text
    assert "LDS bank-conflict cycles / LDS-active cycles: 2.00" in text
    assert "* `cmd b`" in text
    with pytest.raises(KeyError):
        P.summarize_counters([str(tmp_path / "b")], str(out), "k_gemm", ["c"])
