"""Host-side logic of bench.py (CPU only): the one-GPU refusal and the HBM-traffic gate."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_reported_only_for_the_measured_kernel(tmp_path):
    rec = dict(workload="w", alpha=1.0, tiles=10, bytes_per_launch=123.0, attn_source_sha256=bench.attn_source_sha256())
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(path), "w", 1.0, 10) == 123.0
    assert bench.measured_traffic(str(path), "w", 1.25, 10) is None      # another setting
    assert bench.measured_traffic(str(path), "w", 1.0, 11) is None       # another selection
    assert bench.measured_traffic(str(path), "v", 1.0, 10) is None       # another workload
    path.write_text(json.dumps(dict(rec, attn_source_sha256="0" * 64)))
    assert bench.measured_traffic(str(path), "w", 1.0, 10) is None       # counters of another kernel version
    assert bench.measured_traffic(str(tmp_path / "missing.json"), "w", 1.0, 10) is None


def test_committed_traffic_record_is_complete():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        tr = json.load(fh)
    for key in ("workload", "alpha", "tiles", "fetch_kib", "write_kib", "fetch_scale", "write_scale",
                "bytes_per_launch", "attn_source_sha256"):
        assert key in tr, key
    expect = tr["fetch_kib"] * 1024 * tr["fetch_scale"] + tr["write_kib"] * 1024 * tr["write_scale"]
    assert abs(expect - tr["bytes_per_launch"]) <= 1e-6 * expect
