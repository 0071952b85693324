"""bench.py on the GPU, briefly: its last stdout line is one JSON object with
the keys and types of the benchmark contract (metric, value, unit, n_gpus,
steps, warmup, ms_per_step, higher_is_better, scaling, vs_baseline, dtype,
data, config with the workload, and the roofline of the dominant kernel with
frac = achieved / peak)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--secondary", "c3", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    line = r.stdout.strip().splitlines()[-1]
    d = json.loads(line)
    for k, t in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                 ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                 ("dtype", str), ("data", str), ("config", dict), ("roofline", dict)]:
        assert isinstance(d[k], t), k
    assert "vs_baseline" in d
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
    assert d["scaling"] in ("weak", "strong") and d["higher_is_better"] is True
    assert d["config"]["workload"]
    rl = d["roofline"]
    assert rl["bound"] in ("mfma", "hbm", "alu") and rl["unit"] in ("TFLOP/s", "GB/s")
    assert rl["achieved"] > 0 and rl["peak"] > 0
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-9
    assert rl["traffic"] is None or rl["traffic"] > 0
    assert "c3" in d.get("secondary", {})
