"""The benchmark's JSON line on the GPU (a short run through `bench.py` itself):

- one line with the contract's keys, `value` equal to the workload's FLOPs over
  `ms_per_step`, and the settle phase recorded;
- the settle phase runs the call for at least the requested device time, with a launch
  count different from the timed steps (so that a kernel trace can tell them apart).
"""
import json
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

pytestmark = pytest.mark.gpu


def test_bench_line_contract_and_settle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[bench] workload 2, 8 steps, 2 warm-up, 30 ms settle", flush=True)
    r = subprocess.run([sys.executable, "bench.py", "--steps", "8", "--warmup", "2", "--settle-ms", "30",
                        "--no-others", "--no-cpu-baseline"], cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip().startswith("{")]
    assert len(lines) == 1
    j = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "settle"):
        assert key in j, key
    assert j["n_gpus"] == 1 and j["steps"] == 8 and j["warmup"] == 2
    from exact_attention_forward_fwd_amd.workloads import WORKLOADS
    w = WORKLOADS[2]
    assert j["config"]["workload"] == w.name
    assert abs(j["value"] - w.flops / (j["ms_per_step"] * 1e-3) / 1e12) <= 0.02 * j["value"]
    assert j["settle"]["min_device_ms"] == 30 and j["settle"]["device_ms"] >= 30
    assert j["settle"]["launches"] > 0 and j["settle"]["launches"] != j["steps"]
    rf = j["roofline"]
    assert rf["bound"] == "mfma" and 0 < rf["frac"] < 1 and rf["peak"] == 2516.6
