"""Host logic of the profiler summaries (no GPU): rocprofv3 CSV parsing, the
byte-counter calibration of the traffic record, the source-hash check that
retires a record once the kernels change, and the matrix-core summary."""
import csv
import json

import pytest

from gemv_nibble_unpack_amd import profiling as P

HDR = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
       "Start_Timestamp", "End_Timestamp"]


def _counters(d, rows):
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HDR)
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow([i, i, kernel, counter, value, 1000 * i, 1000 * i + 500])


def test_trace_summary(tmp_path):
    d = tmp_path / "t"
    d.mkdir()
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for ns in (4000, 5000, 6000):
            w.writerow(["k_gemv", 0, ns])
        w.writerow(["copy", 0, 1000])
    out = tmp_path / "s.md"
    P.summarize_trace(str(d), str(out), "cmd")
    text = out.read_text()
    assert "`k_gemv` | 3 | 5.00 | 5.00 | 4.00 |" in text
    assert text.index("k_gemv") < text.index("copy")           # by total time
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
