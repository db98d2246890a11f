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
    """The stored counter run: per kernel FETCH_SIZE / WRITE_SIZE (KiB counts) scaled by the copy
    calibration; the stages and the attention launch add up from the kernels."""
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        tr = json.load(fh)
    for key in ("workload", "alpha", "tiles", "sources", "calibration", "kernels", "stages", "bytes_per_launch",
                "attn_source_sha256"):
        assert key in tr, key
    cal = tr["calibration"]
    per_stage = {}
    for name, kv in tr["kernels"].items():
        b = kv["fetch_kib"] * cal["fetch_bytes_per_count"] + kv["write_kib"] * cal["write_bytes_per_count"]
        assert abs(b - kv["bytes"]) <= 1e-4 * b + 1.0, name
        per_stage[kv["stage"]] = per_stage.get(kv["stage"], 0.0) + kv["bytes"]
    for st, b in tr["stages"].items():
        assert abs(per_stage[st] - b) <= 1e-4 * b + 8.0, st
    attn = [kv["bytes"] for name, kv in tr["kernels"].items() if name.startswith("attn_q64_kernel<false")]
    assert len(attn) == 1 and abs(attn[0] - tr["bytes_per_launch"]) <= 1e-4 * attn[0]


def test_stage_counter_bytes_gate(tmp_path):
    """Route / select counter bytes are reported only while their own source is unchanged."""
    path = tmp_path / "traffic.json"
    srcs = {"attn.hip": bench.source_sha256("attn.hip"), "route.hip": bench.source_sha256("route.hip"),
            "select.hip": "0" * 64}
    rec = dict(workload="w", alpha=1.0, tiles=10, sources=srcs, stages={"route": 5, "select": 7, "attn": 9})
    path.write_text(json.dumps(rec))
    assert bench.measured_stage_bytes(str(path), "w", 1.0, 10) == {"route": 5, "attn": 9}
    assert bench.measured_stage_bytes(str(path), "w", 1.0, 11) == {}
    sh = type("S", (), dict(batch=1, h_q=4, h_kv=2, n=1024, d=64, n_blocks=8))()
    res = dict(pe_heads=1, stage_ms={"route": 1.0, "select": 2.0})
    rates = bench.stage_rates(sh, res, {"route": 4e9, "attn": 1.0})
    assert rates["route_counter_gbs"] == 4000.0 and "select_counter_gbs" not in rates
