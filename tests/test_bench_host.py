"""Host logic of bench.py, on the CPU: the one-GPU guard, the algorithmic byte counts behind the
roofline figure, and the gate that reports counted HBM traffic only for the profiled sources."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_decode_bytes_per_launch():
    # a record is 32 u32 words of indices plus one fp16 norm; 4 KV heads, K and V
    per_pos = 4 * 2 * (32 * 4 + 2)
    assert per_pos == 1040 == bench.TQ4_BYTES_PER_POS_LAYER
    # one request of 212,992 positions in 256-position pages, 24 bf16 query heads: the records,
    # the query row and the output row, 832 page-table entries and the length
    assert bench.decode_algorithmic_bytes([212992], 256, 24) == (
        212992 * per_pos + 24 * 256 * 2 * 2 + 832 * 4 + 4)
    # a partial last page still costs its page-table entry
    assert bench.decode_algorithmic_bytes([257], 256, 1) == 257 * per_pos + 256 * 4 + 2 * 4 + 4
    # two requests: per-request query, output, table and length
    two = bench.decode_algorithmic_bytes([131072, 98304], 256, 24)
    assert two == (229376 * per_pos + 2 * 24 * 256 * 4 + (512 + 384) * 4 + 2 * 4)
    # the fused append: fp32 K and V of the new token in, two records out, one slot index
    assert bench.append_bytes(1, 4) == 4 * 2 * (256 * 4 + 130) + 4


def test_traffic_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    got = bench.measured_traffic()
    assert got is not None and got > bench.decode_algorithmic_bytes([212992], 256, 24)
    # a changed source no longer matches the summary's hash: no counted traffic is reported
    copies = []
    for f in bench.DECODE_SOURCES:
        dst = tmp_path / os.path.basename(f)
        dst.write_bytes(open(os.path.join(ROOT, f), "rb").read())
        copies.append(str(dst))
    monkeypatch.setattr(bench, "DECODE_SOURCES", copies)
    assert bench.measured_traffic() == got
    with open(copies[0], "ab") as fh:
        fh.write(b"\n// edited\n")
    assert bench.measured_traffic() is None
