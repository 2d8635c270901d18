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
    assert "experts" in cb["sample"] and "fp32" in cb["sample"] and cb["precision"] == "fp32"
    assert cb["cpu_model"] and cb["blas"] and cb["host_cpus"] >= 1


def test_roofline_bound_and_algorithmic_bytes():
    # Mixtral-like fwd sits far above the ridge point (MFMA-bound); the stress
    # accumulate far below it (HBM-bound); bytes follow the stated formulas
    M, N, K, E = 16384, 14336, 4096, 8
    assert bench.algorithmic_bytes("fwd", M, N, K, E, E) == 2 * (M * K + E * N * K + M * N)
    assert bench.algorithmic_bytes("wgrad_fp32_accumulate", M, N, K, E, E) == 2 * (M * N + M * K) + 8 * E * N * K
    r = bench.roofline_of("fwd", 1.5, M, N, K, E, E)
    assert r["bound"] == "mfma" and abs(r["roofline_frac"] - r["tflops"] / bench.PEAK_BF16_TFLOPS) < 1e-3
    M, N, K, E = 65536, 2048, 7168, 256
    r = bench.roofline_of("wgrad_fp32_accumulate", 6.0, M, N, K, E, E)
    assert r["bound"] == "hbm" and abs(r["roofline_frac"] - r["hbm_gbs"] / bench.PEAK_HBM_GBS) < 1e-3
