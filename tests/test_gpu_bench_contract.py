"""bench.py end to end on a small workload: one JSON line with the fields the
measurement reports, from the HIP library (a child process, the same command a
user runs)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_json_line():
    print("[case] bench.py --config 2 --steps 3 --warmup 1 --no-peaks --no-cpu-baseline", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "2",
                        "--steps", "3", "--warmup", "1", "--no-peaks", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["config"]["workload"] == "switch-base-8e"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert abs(d["value"] - 4096 / (d["ms_per_step"] * 1e-3)) <= 1e-3 * d["value"]
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma") and 0 < rf["frac"] < 1.5
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-3)
    # every stage of the forward was timed, and the stages add up to about a step
    assert set(d["stage_ms"]) >= {"router", "assign", "gemm1_relu", "gemm2_combine"}
    assert d["dispatch_hbm_frac"] is not None and d["combine_hbm_frac"] is not None
    assert d["loads"]["min"] >= 0 and d["kept_assignments"] + d["dropped_assignments"] == 4096
