"""Host logic of bench.py (no GPU): the one-GPU guard and the rule that the
row-pass HBM traffic is reported only from a counter record taken on the
current kernel sources and workload."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, cwd=ROOT, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_traffic_only_from_a_record_of_the_current_sources(tmp_path, monkeypatch):
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.traffic_for("mid") is None  # no record
    sha = bench.kernel_source_sha()
    rec.write_text(json.dumps({"kernel_src_sha": sha, "workload": "mid", "bytes_per_launch": 123}))
    assert bench.traffic_for("mid") == 123
    assert bench.traffic_for("long") is None  # another workload
    rec.write_text(json.dumps({"kernel_src_sha": "0" * 16, "workload": "mid", "bytes_per_launch": 123}))
    assert bench.traffic_for("mid") is None  # taken on other kernel code


def test_source_hash_follows_the_kernel_sources(tmp_path, monkeypatch):
    a = tmp_path / "a.hip"
    a.write_text("x")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ("a.hip",))
    h1 = bench.kernel_source_sha()
    a.write_text("y")
    assert bench.kernel_source_sha() != h1


def test_committed_record_names_the_row_pass_of_the_main_workload():
    with open(os.path.join(ROOT, "profiles", "bob_pass1_traffic.json")) as f:
        rec = json.load(f)
    assert rec["workload"] == "mid" and "bob_pass1_ws_kernel" in rec["kernel"]
    assert rec["bytes_per_launch"] > 0
