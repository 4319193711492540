"""bench.py end to end on the GPU (tiny preset): the one JSON line it prints carries every
field of the reporting contract with consistent values."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line_tiny():
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "tiny",
           "--steps", "3", "--warmup", "1", "--cpu-seconds", "5"]
    print(f"\n[case] {' '.join(cmd[2:])}", flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    print(f"  value={d['value']} {d['unit']} roofline={d['roofline']}", flush=True)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["unit"] == "solves/s" and d["higher_is_better"] is True
    assert (d["n_gpus"], d["steps"], d["warmup"]) == (1, 3, 1)
    assert d["scaling"] == "weak" and d["vs_baseline"] is None
    assert d["dtype"] == "f32" and d["data"] == "synthetic"
    assert d["config"]["workload"] == "tiny"
    # value is whole-job throughput over the timed steps
    assert d["value"] > 0
    assert d["value"] == pytest.approx(d["solves_per_step"] * 1000.0 / d["ms_per_step"],
                                       rel=2e-3)
    roof = d["roofline"]
    assert roof["bound"] in ("hbm", "mfma", "alu")
    assert roof["unit"] == ("GB/s" if roof["bound"] == "hbm" else "TFLOP/s")
    assert roof["achieved"] > 0 and roof["peak"] > 0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    assert "traffic" in roof
    cpu = d["cpu_baseline"]
    assert cpu is not None and cpu["kind"] == "oracle" and cpu["value"] > 0
    assert cpu["unit"] == "solves/s" and cpu["cores"] >= 1 and cpu["sample"]
