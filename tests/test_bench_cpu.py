"""CPU checks of bench.py's host logic: the one-GPU contract and the traffic
record's tie to the kernel sources (no GPU is touched)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_is_reported_only_for_the_recorded_sources(tmp_path, monkeypatch):
    rec = json.load(open(bench.TRAFFIC_FILE))
    assert bench.measured_traffic() in (None, rec["traffic_bytes"])
    # the same record against other sources: no traffic figure
    src = tmp_path / "kernel.hip"
    src.write_text("// another kernel\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    assert bench.measured_traffic() is None
    # a record taken for exactly these sources: its figure
    import hashlib
    h = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    other = tmp_path / "traffic.json"
    other.write_text(json.dumps(dict(rec, source_sha256_16=h)))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(other))
    assert bench.measured_traffic() == rec["traffic_bytes"]

