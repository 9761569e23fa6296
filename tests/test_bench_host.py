"""Host-side logic of bench.py (CPU only): the per-launch traffic computed
from rocprofv3 counter files with the copy-kernel calibration, the
algorithmic byte counts, and the refusal of more than one GPU."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _counter_csv(path, counter, rows):
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_alg_bytes_of_the_batched_workload():
    total, stats = bench.alg_bytes(64, 7, 151936, 3, 2)
    assert stats == 2 * 64 * 8 * 151936 * 2 + 64 * 7 * 4 + 64 * 4 == 311166976
    assert total > stats


def test_traffic_from_counters_uses_the_copy_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    copy_bytes = (bench.alg_bytes(64, 7, 151936, 3, 2)[0] // 8) * 4
    # the copy kernel's FETCH reads half its bytes, WRITE reads all of them
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [
        ("void at::native::neg_kernel_cuda(...)", copy_bytes / 2 / 1024),
        ("void sv::k_stats<unsigned short, 4>(sv::Params)", 1000.0),
        ("void sv::k_stats<unsigned short, 4>(sv::Params)", 3000.0),
        ("void sv::k_decide<unsigned short, 4>(sv::Params)", 500.0),
        ("void other_kernel(int)", 9e9)])
    _counter_csv(write, "WRITE_SIZE", [
        ("void at::native::neg_kernel_cuda(...)", copy_bytes / 1024),
        ("void sv::k_stats<unsigned short, 4>(sv::Params)", 10.0),
        ("void sv::k_decide<unsigned short, 4>(sv::Params)", 2.0)])
    bench.write_traffic(str(fetch), str(write))
    out = json.load(open(tmp_path / "traffic.json"))
    assert out["fetch_scale"] == pytest.approx(2.0)
    assert out["write_scale"] == pytest.approx(1.0)
    assert out["fetch_bytes"] == pytest.approx(2000.0 * 1024 * 2.0)   # mean of 1000 and 3000 KiB
    assert out["write_bytes"] == pytest.approx(10.0 * 1024)
    assert out["k_decide"]["fetch_bytes"] == pytest.approx(500.0 * 1024 * 2.0)
    assert out["kernel_hash"] == bench.kernel_hash()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stdout
