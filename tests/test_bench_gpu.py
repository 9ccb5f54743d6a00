"""The benchmark's output line on a GPU: one JSON object with the fields its
readers parse, the roofline of the scoring kernel and the path, and the
configuration it names.  A short run (3 timed steps) in a child process."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_the_contract_fields():
    print("bench: qwen3_8b_32k, --steps 3 --warmup 1 --no-cpu-baseline", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=100, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "path_hbm"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "seq-decode-steps/s" and d["higher_is_better"] is True
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # throughput is the batch over the step time
    assert abs(d["value"] - d["config"]["batch"] / (d["ms_per_step"] * 1e-3)) <= 0.01 * d["value"]
    assert d["config"]["workload"] == "qwen3_8b_32k" and d["dtype"] == "bf16"
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["algorithmic_bytes"] == 1_075_052_608
    assert d["path_hbm"]["algorithmic_bytes"] == 1_210_777_664
    assert "cpu_baseline" not in d or d["cpu_baseline"] is None
