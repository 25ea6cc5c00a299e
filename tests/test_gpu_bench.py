"""The JSON line bench.py prints, on a short run of the default workload:
every key of the contract with a consistent roofline object and the oracle
baseline beside it."""
import io
import json
import sys

import pytest

pytestmark = pytest.mark.gpu


def _run(argv):
    import bench
    old_argv, old_out = sys.argv, sys.stdout
    buf = io.StringIO()
    sys.argv = ["bench.py"] + argv
    sys.stdout = buf
    try:
        bench.main()
    finally:
        sys.argv, sys.stdout = old_argv, old_out
    lines = [l for l in buf.getvalue().splitlines() if l.startswith("{")]
    assert len(lines) == 1
    return json.loads(lines[0])


def test_bench_json_contract():
    print("bench contract: default workload, 5 steps", flush=True)
    d = _run(["--steps", "5", "--warmup", "2", "--cpu-seconds", "1"])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["vs_baseline"] is None and d["data"] == "synthetic"
    assert "workload" in d["config"]
    r = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in r, key
    assert r["bound"] in ("hbm", "mfma", "alu")
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
    # the value is outputs per second of the timed calls
    cfg = d["config"]
    want = cfg["B"] * cfg["H"] * cfg["N"] / (d["ms_per_step"] * 1e-3)
    assert abs(d["value"] - want) / want < 1e-3
