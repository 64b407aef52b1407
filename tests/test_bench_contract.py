"""bench.py's host-side contract, without a GPU: the one-GPU refusal, the
committed HBM-traffic records, and the rule that a record taken on other
kernel sources is reported as unknown (null) rather than reused."""

import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


RECORDS = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json")))


def test_traffic_records_exist():
    names = {os.path.basename(p) for p in RECORDS}
    assert "decode_partition_llama_gqa4k_bf16_traffic.json" in names


@pytest.mark.parametrize("path", RECORDS, ids=[os.path.basename(p) for p in RECORDS])
def test_traffic_record_is_consistent(path):
    with open(path) as f:
        rec = json.load(f)
    for key in ("kernel", "workload", "kernel_source_sha256_16", "hbm_read_bytes_per_launch",
                "hbm_write_bytes_per_launch", "hbm_bytes_per_launch", "algorithmic_read_bytes_per_launch",
                "algorithmic_write_bytes_per_launch", "copy_calibration", "commands"):
        assert key in rec, key
    h = rec["kernel_source_sha256_16"]
    assert len(h) == 16 and all(c in "0123456789abcdef" for c in h)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(rec["hbm_read_bytes_per_launch"] +
                                                        rec["hbm_write_bytes_per_launch"])
    # every kernel reads at least its algorithmic bytes (whole blocks, L2 misses) and not wildly more
    ratio = rec["hbm_read_bytes_per_launch"] / rec["algorithmic_read_bytes_per_launch"]
    assert 0.99 <= ratio <= 2.5, ratio
    cal = rec["copy_calibration"]
    assert cal["fetch_scale"] == pytest.approx(cal["copy_bytes"] / (cal["fetch_kib"] * 1024))
    assert cal["write_scale"] == pytest.approx(cal["copy_bytes"] / (cal["write_kib"] * 1024))
    assert all(c.startswith("rocprofv3 --pmc ") for c in rec["commands"])


def test_stale_traffic_record_reads_as_unknown(monkeypatch):
    prefix = "decode_partition"
    assert len(bench.kernel_source_hash(prefix)) == 16
    monkeypatch.setattr(bench, "kernel_source_hash", lambda p="decode_partition": "0" * 16)
    assert bench.load_traffic("llama_gqa4k_bf16", prefix) is None
    assert bench.load_traffic("no_such_workload", prefix) is None
