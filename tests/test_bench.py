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


def test_profile_counter_parsing(tmp_path):
    # the profiling harness sums a counter over the dispatches of a call's
    # kernels (not the spectrum set-up or the runtime's copies)
    d = tmp_path / "pmc" / "host" / "123"
    d.mkdir(parents=True)
    hdr = ('"Correlation_Id","Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
    body = [
        '1,1,"__amd_rocclr_copyBuffer","SQ_INSTS_VALU",5.0',
        '2,2,"fftconv::stockham_kernel(float2 const*)","SQ_INSTS_VALU",7.0',
        '3,3,"void fftconv::row_kernel<2, 32, false, false>(fftconv::RowParams)","SQ_INSTS_VALU",100.0',
        '4,4,"void fftconv::row_kernel<2, 32, false, false>(fftconv::RowParams)","SQ_INSTS_VALU",50.0',
        '4,4,"void fftconv::row_kernel<2, 32, false, false>(fftconv::RowParams)","GRBM_GUI_ACTIVE",8.0',
        '5,5,"fftconv::stream_copy_kernel(unsigned int const*)","SQ_INSTS_VALU",1.0',
    ]
    (d / "pmc_counter_collection.csv").write_text(hdr + "\n".join(body) + "\n")
    got = bench._counters(str(tmp_path / "pmc"), bench._is_call_kernel)
    assert got == {"SQ_INSTS_VALU": 150.0, "GRBM_GUI_ACTIVE": 8.0}
    cp = bench._counters(str(tmp_path / "pmc"), lambda n: "stream_copy" in n)
    assert cp == {"SQ_INSTS_VALU": 1.0}


def test_profile_counter_groups_fit_one_pass():
    # rocprofv3 does not split counters over passes: at most 8 SQ and 2 GRBM
    # counters per pass, and the TCC byte counters each in a pass of their own
    for group in bench.PMC_PASSES:
        sq = [c for c in group if c.startswith("SQ_")]
        grbm = [c for c in group if c.startswith("GRBM_")]
        assert len(sq) <= 8 and len(grbm) <= 2
        if "FETCH_SIZE" in group or "WRITE_SIZE" in group:
            assert len(group) == 1
