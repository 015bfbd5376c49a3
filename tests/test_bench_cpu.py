"""bench.py's host-side behaviour (no GPU needed): more than one GPU is
refused with a message, and the traffic record is computed from counter
files as the scaled sum of FETCH_SIZE and WRITE_SIZE."""

import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counter_dir(tmp_path, name, kernel, counter, values):
    d = tmp_path / name
    d.mkdir()
    with open(d / "p_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for v in values:
            w.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": v})
    return str(d)


def test_traffic_record_from_counters(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    k = "void bra::attend_region_kernel<...>(RegionArgs)"
    c = "__amd_rocclr_copyBuffer"
    dirs = [_counter_dir(tmp_path, "f", k, "FETCH_SIZE", [1000.0, 1200.0]),
            _counter_dir(tmp_path, "w", k, "WRITE_SIZE", [500.0]),
            _counter_dir(tmp_path, "cf", c, "FETCH_SIZE", [131072.0]),     # a copy of 256 MiB
            _counter_dir(tmp_path, "cw", c, "WRITE_SIZE", [262144.0])]
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "st1", "--traffic-from", *dirs])
    assert bench.write_traffic(bench.parse()) == 0
    rec = json.load(open(out))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["bytes_per_launch"] == 1100.0 * 1024 * 2.0 + 500.0 * 1024 * 1.0
    assert rec["workload"] == "st1" and rec["kernel_sha"] == bench.kernel_sha()
