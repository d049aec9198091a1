"""Host logic of the benchmark (no GPU): the algorithmic byte counts its
roofline divides by, and its refusal of more than one GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_bytes_w4a16_4096():
    # packed codes 8,388,608 + fp16 scales 262,144 + uint8 zeros 131,072
    # + fp16 activation row 8,192 + fp16 output row 8,192
    assert bench.decode_bytes(1, 4096, 4096) == 8_798_208


def test_prefill_bytes_w4a8_2048_11008_4096():
    # packed codes 22,544,384 + fp32 w_scale 44,032 + int8 A 8,388,608
    # + fp32 a_scale 8,192 + fp16 bias 22,016 + fp16 C 45,088,768
    assert bench.prefill_bytes(2048, 11008, 4096) == 76_096_000


def test_timed_calls_read_cold_weights():
    # Between two reads of one weight copy inside a timed region, more bytes
    # than the last-level cache holds pass through memory: the flush before
    # the region, or the other copies when the rotation comes round. This
    # holds at the driver's step count and at the defaults, for the decode
    # and the prefill copies.
    for copy_bytes in (bench.decode_bytes(1, 4096, 4096), 4096 * 11008 // 2 + 3 * 11008 * 32,
                       11008 * 4096 // 2):
        R = bench.rotation(copy_bytes)
        assert R * copy_bytes >= bench.ROTATE_BYTES
        for steps in (1, 5, 20, 50, 200, 1000):
            assert bench.cold_gap_bytes(steps, R, copy_bytes) > 2 * bench.LLC_BYTES
    assert bench.FLUSH_BYTES >= 4 * bench.LLC_BYTES
    assert bench.PREFILL_MIN_STEPS >= 50


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""
