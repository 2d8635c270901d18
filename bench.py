#!/usr/bin/env python3
"""Benchmark of the deterministic ragged BF16 grouped GEMM on one MI355X.

One step = one pass of the whole hot path over one batch of the workload:
fwd (Y = X W^T per group), dgrad (dX = G W per group) and wgrad with the fused
fp32 accumulate into main_grad (dW = G^T X per expert, added into main_grad),
i.e. the expert-projection GEMMs of one MoE layer's training step.

Prints ONE JSON line.  `value` is the step's grouped-GEMM throughput in TFLOP/s
(3 x 2*M*N*K algorithmic FLOPs per step over the measured step time), with all
inputs resident in HBM.  `roofline` reports the dominant kernel against the
MI355X dense bf16 MFMA peak; `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload (rank 0 only).

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload mixtral]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (published)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    from workloads import CONFIGS
    ap.add_argument("--workload", default="mixtral", choices=list(CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-autograd", action="store_true",
                    help="skip timing the same step through the autograd wrapper")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times): the reference kernel "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def copy_calibration(mib: int) -> None:
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "reps": 5}), flush=True)


def kernel_source_digest() -> str:
    import hashlib
    path = os.path.join(ROOT, "moe_ragged_bf16_amd", "csrc", "grouped_gemm_kernels.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3
    PMC summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy kernel), or None
    if there is none or the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_digest():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(d, target_s: float):
    """Time the CPU oracle (fp64, as it stands) on whole experts of the workload,
    in expert order, until about target_s seconds have been spent."""
    import numpy as np
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1

    def bits(t):
        import torch
        return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    sizes = d["sizes"]
    N, K = d["N"], d["K"]
    flops = 0.0
    spent = 0.0
    used = []
    passes = 0
    while spent < target_s:  # whole experts in order, again from the first if time is left
        passes += 1
        s = 0
        for e, m in enumerate(sizes):
            m = int(m)
            t0, t1 = s, s + m
            s = t1
            if m == 0:
                continue
            X = bits(d["x"][t0:t1])
            G = bits(d["g"][t0:t1])
            W = bits(d["w"][e:e + 1])
            offs = np.array([m], dtype=np.int32)
            c0 = time.perf_counter()
            oracle.fwd(X, W, offs)
            oracle.dgrad(G, W, offs)
            oracle.wgrad(G, X, offs)
            spent += time.perf_counter() - c0
            flops += 3 * 2.0 * m * N * K
            if passes == 1:
                used.append((e, m))
            if spent >= target_s:
                break
    rows = sum(m for _, m in used)
    what = (f"all {len(used)} non-empty experts ({rows} rows), {passes} passes" if passes > 1 else
            f"experts {used[0][0]}..{used[-1][0]} ({len(used)} experts, {rows} rows)")
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{what} of the workload, fwd+dgrad+wgrad in fp64 NumPy, {spent:.1f} s",
    }


def time_autograd(mdg, d, steps: int, warmup: int, direct_ms: float, flop_op: float) -> dict:
    """The same step through cake_grouped_det_mm: forward, then a backward with
    the fused fp32 accumulate into w.main_grad (Megatron placeholder for w.grad).
    Timed after the main measurement; it does not enter `value`."""
    import time as _time

    import torch

    x = d["x"].detach().requires_grad_()
    w = d["w"].detach().requires_grad_()
    w.main_grad = d["main_grad"]
    w.grad_added_to_main_grad = False
    g, offs = d["g"], d["offs"]

    def one():
        x.grad = None
        w.grad = None
        y = mdg.cake_grouped_det_mm(x, w, offs, fuse_wgrad_accumulation=True)
        y.backward(g)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = _time.perf_counter()
    start.record()
    for _ in range(steps):
        one()
    stop.record()
    torch.cuda.synchronize()
    wall = _time.perf_counter() - t0
    ms = start.elapsed_time(stop) / steps
    return {"ms_per_step": round(ms, 4), "tflops": round(3 * flop_op / (ms * 1e-3) / 1e12, 1),
            "overhead_vs_direct_pct": round(100.0 * (ms / direct_ms - 1.0), 2),
            "host_wall_ms_per_step": round(1e3 * wall / steps, 4),
            "step": "cake_grouped_det_mm forward + backward: dgrad, wgrad fused into fp32 w.main_grad, "
                    "zero fill of the padding rows of Y and dX, placeholder w.grad"}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "this benchmark has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_ragged_bf16_amd as mdg
    from workloads import CONFIGS, make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = CONFIGS[args.workload]
    d = make_inputs(args.workload, seed=0, device=dev, tensors=("x", "w", "g", "main_grad"))
    M, N, K, E = d["M"], d["N"], d["K"], d["E"]
    x, w, g, offs, mg = d["x"], d["w"], d["g"], d["offs"], d["main_grad"]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(mdg.wgrad_workspace_bytes(M, N, K, E), 256), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(mdg.fwd_workspace_bytes(M, N, K, E), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(mdg.dgrad_workspace_bytes(M, N, K, E), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        mdg.grouped_det_gemm_fwd(x, w, offs, out=y, workspace=ws_f)
        if ev is not None:
            ev[1].record()
        mdg.grouped_det_gemm_dgrad(g, w, offs, out=dx, workspace=ws_d)
        if ev is not None:
            ev[2].record()
        mdg.grouped_det_gemm_wgrad(g, x, offs, out=mg, accumulate=True, workspace=ws)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(events[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    op_ms = {
        "fwd": float(np.mean([e[0].elapsed_time(e[1]) for e in events])),
        "dgrad": float(np.mean([e[1].elapsed_time(e[2]) for e in events])),
        "wgrad_fp32_accumulate": float(np.mean([e[2].elapsed_time(e[3]) for e in events])),
    }
    flop_op = 2.0 * M * N * K
    value = 3 * flop_op / (ms_per_step * 1e-3) / 1e12

    # bitwise rerun check of the measured kernels (outputs must not change)
    y_ref = y.clone()
    dx_ref = dx.clone()
    mdg.grouped_det_gemm_fwd(x, w, offs, out=y, workspace=ws_f)
    mdg.grouped_det_gemm_dgrad(g, w, offs, out=dx, workspace=ws_d)
    torch.cuda.synchronize()
    rerun_ok = bool(torch.equal(y.view(torch.int16), y_ref.view(torch.int16)) and
                    torch.equal(dx.view(torch.int16), dx_ref.view(torch.int16)))
    if not rerun_ok:
        print("bitwise rerun check FAILED", file=sys.stderr)
        sys.exit(1)

    sizes = d["sizes"]
    e_ne = int((sizes > 0).sum())
    ops = {}
    for name, ms in op_ms.items():
        tf = flop_op / (ms * 1e-3) / 1e12
        ops[name] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                     "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1)}
    # dominant kernel: the op with the largest average launch time
    dom = max(op_ms, key=op_ms.get)
    achieved = flop_op / (op_ms[dom] * 1e-3) / 1e12
    # algorithmic HBM bytes per launch: each operand read once, outputs written once
    # (W only for non-empty experts; main_grad read and written by the accumulate)
    alg_bytes = {
        "fwd": 2 * (M * K + e_ne * N * K + M * N),
        "dgrad": 2 * (M * N + e_ne * N * K + M * K),
        "wgrad_fp32_accumulate": 2 * (M * N + M * K) + 8 * E * N * K,
    }
    kernel_name = {"fwd": "fwd", "dgrad": "dgrad", "wgrad_fp32_accumulate": "wgrad"}[dom]
    traffic = measured_traffic(args.workload, kernel_name)
    # the kernel's bound: MFMA above the ridge point (peak FLOP/s / peak bytes/s),
    # HBM below it (then achieved and peak are algorithmic bytes per second)
    intensity = flop_op / alg_bytes[dom]
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if intensity >= ridge:
        bound, ach, peak, unit = "mfma", achieved, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        bound, unit, peak = "hbm", "GB/s", PEAK_HBM_GBS
        ach = alg_bytes[dom] / (op_ms[dom] * 1e-3) / 1e9
    roofline = {"bound": bound, "achieved": round(ach, 1), "peak": peak,
                "unit": unit, "frac": round(ach / peak, 4),
                "traffic": traffic, "kernel": dom,
                "tflops": round(achieved, 1), "ridge_flop_per_byte": round(ridge, 1),
                "flops_per_launch": flop_op,
                "algorithmic_bytes_per_launch": alg_bytes[dom],
                "arithmetic_intensity": round(flop_op / alg_bytes[dom], 1),
                "hbm_gbs_at_algorithmic_bytes": round(alg_bytes[dom] / (op_ms[dom] * 1e-3) / 1e9, 1)}

    autograd = None
    if not args.no_autograd:
        autograd = time_autograd(mdg, d, args.steps, max(args.warmup, 1), ms_per_step, flop_op)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(d, args.cpu_seconds)

    line = {
        "metric": "grouped GEMM TFLOP/s (fwd/dgrad/wgrad) + % of bf16 MFMA peak, 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded routing and N(0,1) operands, bf16)",
        "config": {"workload": cfg.name, "description": cfg.description, "E": E, "K": K, "N": N,
                   "sum_m": M, "nonempty_experts": e_ne,
                   "step": "fwd + dgrad + wgrad(fp32, fused accumulate into main_grad)"},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 1),
        "ops": ops,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "autograd": autograd,
        "rerun_bitwise": rerun_ok,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
