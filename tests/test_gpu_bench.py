"""bench.py keeps its output contract (GPU): one JSON line with the metric, the
whole-step throughput, the roofline of the dominant kernel and the oracle's
CPU baseline, for a row-wise (HBM-bound) step and for the chunked-prefill
(matrix-core-bound) step."""
import json
import math
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("cfg,bound,unit", [(1, "hbm", "GB/s"), (3, "mfma", "TFLOP/s")])
def test_bench_prints_one_json_line(cfg, bound, unit):
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--config", str(cfg), "--steps", "3",
           "--warmup", "1", "--cpu-seconds", "0.5", "--no-ceilings"]
    print("running", " ".join(cmd[2:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["vs_baseline"] is None and d["data"] == "synthetic"
    assert d["dtype"] == ("f32" if cfg == 1 else "bf16")
    assert math.isfinite(d["value"]) and d["value"] > 0 and d["unit"] == unit
    assert isinstance(d["config"]["workload"], str) and d["config"]["workload"]
    roof = d["roofline"]
    assert roof["bound"] == bound
    for key in ("achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert math.isfinite(roof["achieved"]) and roof["achieved"] > 0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"])
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0 and cpu["sample"]
    step = d["step_roofline"]
    assert step["t_step_ms"] == pytest.approx(d["ms_per_step"])
    assert 0 < step["frac"] == pytest.approx(step["t_roof_ms"] / step["t_step_ms"])
