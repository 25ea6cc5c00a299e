"""bench.py's contract on the host: one GPU only, and measured HBM traffic is
reported only for the kernel sources the counters were taken on."""
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


def test_traffic_record_requires_the_current_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    cur = bench.kernel_source_hash()
    f.write_text(json.dumps({
        "w_now": {"source_sha1": cur, "traffic_bytes": 1234},
        "w_old": {"source_sha1": "0" * 40, "traffic_bytes": 99}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("w_now") == 1234
    assert bench.measured_traffic("w_old") is None
    assert bench.measured_traffic("absent") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("w_now") is None


def test_source_hash_covers_every_library_source():
    # any edit to a kernel or host source changes the hash
    d = os.path.join(ROOT, "fft_long_convolution_amd", "csrc")
    names = [n for n in os.listdir(d) if n.endswith((".hip", ".cpp", ".h"))]
    assert len(names) >= 5
    assert len(bench.kernel_source_hash()) == 40
