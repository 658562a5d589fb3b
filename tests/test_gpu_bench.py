"""bench.py's output contract, run as a child process on a small batch: one
JSON line with the fields the benchmark promises, self-consistent."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_json_line_with_the_contract_fields():
    print("[case] bench.py --workload tiny_f32 --steps 5 --warmup 2", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny_f32",
                        "--steps", "5", "--warmup", "2", "--cpu-seconds", "0.5",
                        "--no-prior-art"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["data"] == "synthetic" and d["vs_baseline"] is None and d["dtype"] == "f32"
    assert d["config"]["workload"].startswith("tiny_f32")
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["peak"] == 8000.0 and rl["unit"] == "GB/s"
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    # One launch per step: the step's kernel rate is the step rate.
    assert abs(rl["achieved"] - d["value"]) <= 1e-3 * d["value"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["host_cores"] >= cb["cores"] and cb["one_thread"]["value"] > 0
