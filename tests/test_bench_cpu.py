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



def _counter_csv(d, counter, rows):
    d.mkdir(parents=True, exist_ok=True)
    with open(d / "t_counter_collection.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (name, v) in enumerate(rows):
            f.write(f"{i + 1},\"{name}\",{counter},{v}\n")


def test_stage_traffic_record_scales_by_the_copy(tmp_path):
    # FETCH_SIZE reading half of a 1 GiB copy's reads scales by 2, WRITE_SIZE
    # reading it exactly by 1; medians over 8 dispatches of each
    stage = "cq4_65536x512_gather_4096"
    kern = "void bqd::cq_gather_kernel<4, 8, 7, true>(unsigned char const*)"
    copy = "__amd_rocclr_copyBuffer"
    # uploads of the inputs are earlier, small copies: only the last 8 calibrate
    _counter_csv(tmp_path / "f", "FETCH_SIZE",
                 [(copy, 3.0)] * 20 + [(kern, 600.0)] * 8 + [(copy, 524288.0)] * 8)
    _counter_csv(tmp_path / "w", "WRITE_SIZE", [(kern, 8192.0)] * 8 + [(copy, 1048576.0)] * 8)
    bench.stage_traffic_record(stage, str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path))
    rec = json.load(open(tmp_path / "cq_gather_kernel_cq4_65536x512_gather_4096_hbm_traffic.json"))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["read_bytes"] == 600 * 1024 * 2 and rec["write_bytes"] == 8192 * 1024
    assert rec["algorithmic_write_bytes"] == 4 * 4096 * 512
    assert rec["kernel"] == ["void bqd::cq_gather_kernel<4, 8, 7, true>"]
    assert (tmp_path / "cq_gather_kernel_cq4_65536x512_gather_4096_hbm_traffic.md").exists()
