"""bench.py's host-side contract, on the CPU: the one-GPU refusal and the oracle baseline leg."""
import os
import subprocess
import sys

import bench
from workloads import make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""          # no JSON line for a configuration that was not measured


def test_cpu_baseline_leg_times_the_oracle():
    d = make_inputs("tiny", seed=0, device="cpu")
    cb = bench.cpu_baseline(d, 0.05)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert "experts" in cb["sample"] and "fp64" in cb["sample"]
