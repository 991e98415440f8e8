"""bench.py's output contract: one JSON line with the documented fields.  The
refusal of multi-GPU runs is checked on the CPU; a short real run on the GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, timeout=600):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_multi_gpu_request_exits_with_message():
    r = _run("--gpus", "2", timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


@pytest.mark.gpu
def test_short_run_prints_one_contract_line():
    import torch
    if torch.cuda.is_available():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()   # cached blocks of earlier tests go back to the device
    r = _run("--steps", "2", "--warmup", "1", "--skip-cpu-baseline", "--kernel-launches", "4")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.strip().splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["vs_baseline"] is None and d["cpu_baseline"] is None and d["dtype"] == "bf16"
    assert "workload" in d["config"]
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert "traffic" in rf
    # the roofline is the hot kernel with the largest time per forward
    ks = d["kernels"]
    assert {k["name"] for k in ks} >= {"qkv", "out_proj", "fc1", "fc2", "attention", "layernorm"}
    assert all(k["avg_launch_us"] > 0 and k["avg_launch_us_alone"] > 0 for k in ks)
    top = max(ks, key=lambda k: k["us_per_forward"])
    assert rf["kernel"] == top["kernel"]
    assert len(d["repeats_ms_per_step"]) == 5
