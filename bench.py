#!/usr/bin/env python3
"""Benchmark of the deterministic ragged BF16 grouped GEMM on one MI355X.

One step = one pass of the whole hot path over one batch of the workload:
fwd (Y = X W^T per group), dgrad (dX = G W per group) and wgrad with the fused
fp32 accumulate into main_grad (dW = G^T X per expert, added into main_grad),
i.e. the expert-projection GEMMs of one MoE layer's training step.

Prints ONE JSON line.  `value` is the step's grouped-GEMM throughput in TFLOP/s
(3 x 2*M*N*K algorithmic FLOPs per step over the measured step time) on the
Mixtral-like workload, with all inputs resident in HBM.  `roofline` reports the
step's dominant kernel against the MI355X dense bf16 MFMA peak (or HBM below
the ridge point).  `ops` and `configs` follow the per-operation protocol: each
operation alone, a 1 GiB buffer written before every rep to flush the L2s and
the MALL, the median of the HIP-event times; `configs` covers the other
workloads (tiny, fine-grained, skewed, accumulate stress, and the gate_up and
down projection shapes at 4, 8, 16 and 32 experts) that way.
`cpu_baseline` times the fp32 CPU oracle on a bounded sample of the workload.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload mixtral]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (published)
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # FLOP per byte
OPS = ("fwd", "dgrad", "wgrad_bf16", "wgrad_fp32", "wgrad_fp32_accumulate")
OTHER_CONFIGS = ("tiny", "fine", "skewed", "stress",
                 "gate_up_e4", "down_e4", "gate_up_e8", "down_e8",
                 "gate_up_e16", "down_e16", "gate_up_e32", "down_e32")
FLUSH_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    from workloads import CONFIGS
    ap.add_argument("--workload", default="mixtral", choices=list(CONFIGS))
    ap.add_argument("--reps", type=int, default=10,
                    help="timed reps per operation in the per-operation protocol (0: skip it, and the "
                         "host-call latency, e.g. under a profiler)")
    ap.add_argument("--configs", default=",".join(OTHER_CONFIGS),
                    help="comma-separated workloads measured per operation besides --workload "
                         "('none' for none)")
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


def host_info() -> dict:
    """CPU model and the BLAS build NumPy uses (for the CPU baseline)."""
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer')}, " \
                       f"{i.get('architecture')})"
                threads = int(i.get("num_threads", 1))
                break
    except Exception:  # pragma: no cover
        pass
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu_model": model, "blas": blas, "blas_threads": threads or affinity, "host_cpus": affinity}


def cpu_baseline(d, target_s: float, precision: str = "fp32"):
    """Time the CPU oracle (as it stands; fp32 products and sums, the
    accumulation precision of the operation) on whole experts of the workload,
    in expert order, until about target_s seconds have been spent."""
    import numpy as np
    import oracle

    info = host_info()

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
            oracle.fwd(X, W, offs, precision=precision)
            oracle.dgrad(G, W, offs, precision=precision)
            oracle.wgrad(G, X, offs, precision=precision)
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
        "cores": int(info["blas_threads"]),
        "kind": "oracle",
        "sample": f"{what} of the workload, fwd+dgrad+wgrad in {precision} NumPy (BLAS), {spent:.1f} s",
        "precision": precision,
        "cpu_model": info["cpu_model"],
        "blas": info["blas"],
        "host_cpus": info["host_cpus"],
    }


def time_autograd(mdg, d, steps: int, warmup: int, direct_ms: float, flop_op: float) -> dict:
    """The same step through cake_grouped_det_mm: forward, then a backward with
    the fused fp32 accumulate into w.main_grad (Megatron placeholder for w.grad).
    Timed after the main measurement; it does not enter `value`."""
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
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        one()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / steps
    return {"ms_per_step": round(ms, 4), "tflops": round(3 * flop_op / (ms * 1e-3) / 1e12, 1),
            "overhead_vs_direct_pct": round(100.0 * (ms / direct_ms - 1.0), 2),
            "host_wall_ms_per_step": round(1e3 * wall / steps, 4),
            "step": "cake_grouped_det_mm forward + backward: dgrad, wgrad fused into fp32 w.main_grad, "
                    "zero fill of the padding rows of Y and dX, placeholder w.grad"}


def algorithmic_bytes(op: str, M: int, N: int, K: int, E: int, e_ne: int) -> int:
    """HBM bytes one call must move: each operand read once, each output written
    once; W only for experts with rows; dW for every expert (read and written by
    the accumulate)."""
    if op in ("fwd", "dgrad"):
        return 2 * (M * K + e_ne * N * K + M * N)
    per = {"wgrad_bf16": 2, "wgrad_fp32": 4, "wgrad_fp32_accumulate": 8}[op]
    return 2 * (M * N + M * K) + per * E * N * K


def roofline_of(op: str, ms: float, M: int, N: int, K: int, E: int, e_ne: int) -> dict:
    flop = 2.0 * M * N * K
    nbytes = algorithmic_bytes(op, M, N, K, E, e_ne)
    tf = flop / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    if flop / nbytes >= RIDGE:
        bound, frac = "mfma", tf / PEAK_BF16_TFLOPS
    else:
        bound, frac = "hbm", gbs / PEAK_HBM_GBS
    return {"ms": round(ms, 4), "tflops": round(tf, 1), "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1),
            "hbm_gbs": round(gbs, 1), "bound": bound, "roofline_frac": round(frac, 4),
            "flop_per_byte": round(flop / nbytes, 1)}


class Runners:
    """Callables for each operation on one workload's resident tensors, with
    preallocated outputs and workspaces (nothing allocated while timed)."""

    def __init__(self, mdg, torch, d):
        M, N, K, E = d["M"], d["N"], d["K"], d["E"]
        dev = d["x"].device
        self.d = d
        self.mdg = mdg
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        self.dw16 = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
        self.dw32 = torch.empty((E, N, K), dtype=torch.float32, device=dev)
        self.ws = torch.empty(max(mdg.wgrad_workspace_bytes(M, N, K, E), 256), dtype=torch.uint8, device=dev)
        self.ws_f = torch.empty(mdg.fwd_workspace_bytes(M, N, K, E), dtype=torch.uint8, device=dev)
        self.ws_d = torch.empty(mdg.dgrad_workspace_bytes(M, N, K, E), dtype=torch.uint8, device=dev)

    def fwd(self):
        d = self.d
        self.mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"], out=self.y, workspace=self.ws_f)

    def dgrad(self):
        d = self.d
        self.mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"], out=self.dx, workspace=self.ws_d)

    def wgrad_bf16(self):
        d = self.d
        self.mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out=self.dw16, workspace=self.ws)

    def wgrad_fp32(self):
        d = self.d
        self.mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out=self.dw32, workspace=self.ws)

    def wgrad_fp32_accumulate(self, mg):
        d = self.d
        self.mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out=mg, accumulate=True, workspace=self.ws)


def measure_ops(torch, run: Runners, mg, mg0, reps: int, warmup: int, flush) -> dict:
    """Each operation alone: `warmup` untimed calls, then `reps` timed calls, each
    after a 1 GiB write that evicts the L2s and the MALL; the accumulate starts
    every rep from the pristine main_grad (restored before the flush).  HIP
    events on the current stream bracket the call; median, min and mean in ms."""
    out = {}
    for op in OPS:
        fn = (lambda: run.wgrad_fp32_accumulate(mg)) if op == "wgrad_fp32_accumulate" else getattr(run, op)
        for _ in range(warmup):
            fn()
        evs = []
        for r in range(reps):
            if op == "wgrad_fp32_accumulate":
                mg.copy_(mg0)
            flush.fill_(r & 0x7F)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        t = [a.elapsed_time(b) for a, b in evs]
        out[op] = {"median_ms": statistics.median(t), "min_ms": min(t), "mean_ms": statistics.fmean(t)}
    return out


def ops_report(meas: dict, d) -> dict:
    M = int(d["sizes"].sum())
    N, K, E = d["N"], d["K"], d["E"]
    e_ne = int((d["sizes"] > 0).sum())
    rep = {}
    for op, m in meas.items():
        r = roofline_of(op, m["median_ms"], M, N, K, E, e_ne)
        r["min_ms"] = round(m["min_ms"], 4)
        r["mean_ms"] = round(m["mean_ms"], 4)
        rep[op] = r
    return rep


def host_call_latency(torch, mdg, run: Runners, calls: int = 50) -> dict:
    """Host time one call takes to return (validation + enqueue), per call, from a
    synchronised start; the GPU work itself is not waited for."""
    d = run.d
    res = {}
    launch = mdg.prepare_grouped_det_gemm_fwd(d["x"], d["w"], d["offs"], out=run.y, workspace=run.ws_f)
    for name, fn in (("fwd_one_shot", run.fwd), ("wgrad_fp32_one_shot", run.wgrad_fp32),
                     ("fwd_prepared_launch", launch.launch)):
        fn()
        torch.cuda.synchronize()
        per = []
        for _ in range(calls):
            t0 = time.perf_counter()
            fn()
            per.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
        res[name + "_us"] = round(1e6 * statistics.median(per), 2)
    launch.close()
    return res


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
    mg0 = mg.clone()            # pristine main_grad for the rerun checks and the accumulate reps
    run = Runners(mdg, torch, d)
    y, dx = run.y, run.dx
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        run.fwd()
        if ev is not None:
            ev[1].record()
        run.dgrad()
        if ev is not None:
            ev[2].record()
        run.wgrad_fp32_accumulate(mg)
        if ev is not None:
            ev[3].record()

    print(f"bench: {cfg.name} E={E} N={N} K={K} M={M}, {args.warmup} warmup + {args.steps} timed steps",
          file=sys.stderr, flush=True)
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

    # bitwise rerun checks of the measured kernels: fwd and dgrad reproduce their
    # outputs; the fused accumulate from a pristine main_grad reproduces its
    # result and equals main_grad0 + the library's own overwrite dW
    y_ref, dx_ref = y.clone(), dx.clone()
    run.fwd()
    run.dgrad()
    mg.copy_(mg0)
    run.wgrad_fp32_accumulate(mg)
    acc_ref = mg.clone()
    mg.copy_(mg0)
    run.wgrad_fp32_accumulate(mg)
    run.wgrad_fp32()
    torch.cuda.synchronize()
    t = int(d["sizes"].sum())
    rerun = {
        "fwd": bool(torch.equal(y[:t].view(torch.int16), y_ref[:t].view(torch.int16))),
        "dgrad": bool(torch.equal(dx[:t].view(torch.int16), dx_ref[:t].view(torch.int16))),
        "wgrad_fp32_accumulate": bool(torch.equal(mg.view(torch.int32), acc_ref.view(torch.int32))),
        "accumulate_equals_add_of_own_dw": bool(torch.equal(mg.view(torch.int32),
                                                            (mg0 + run.dw32).view(torch.int32))),
    }
    del acc_ref
    rerun_ok = all(rerun.values())
    if not rerun_ok:
        print(f"bitwise rerun check FAILED: {rerun}", file=sys.stderr)
        sys.exit(1)

    e_ne = int((d["sizes"] > 0).sum())
    ops = {}
    for name, ms in op_ms.items():
        tf = flop_op / (ms * 1e-3) / 1e12
        ops[name] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                     "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1)}
    # dominant kernel: the op with the largest average launch time in the timed steps
    dom = max(op_ms, key=op_ms.get)
    achieved = flop_op / (op_ms[dom] * 1e-3) / 1e12
    alg = algorithmic_bytes(dom, M, N, K, E, e_ne)
    kernel_name = {"fwd": "fwd", "dgrad": "dgrad", "wgrad_fp32_accumulate": "wgrad"}[dom]
    traffic = measured_traffic(args.workload, kernel_name)
    # the kernel's bound: MFMA above the ridge point (peak FLOP/s / peak bytes/s),
    # HBM below it (then achieved and peak are algorithmic bytes per second)
    if flop_op / alg >= RIDGE:
        bound, ach, peak, unit = "mfma", achieved, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        bound, unit, peak = "hbm", "GB/s", PEAK_HBM_GBS
        ach = alg / (op_ms[dom] * 1e-3) / 1e9
    roofline = {"bound": bound, "achieved": round(ach, 1), "peak": peak,
                "unit": unit, "frac": round(ach / peak, 4),
                "traffic": traffic, "kernel": dom,
                "tflops": round(achieved, 1), "ridge_flop_per_byte": round(RIDGE, 1),
                "flops_per_launch": flop_op,
                "algorithmic_bytes_per_launch": alg,
                "arithmetic_intensity": round(flop_op / alg, 1),
                "hbm_gbs_at_algorithmic_bytes": round(alg / (op_ms[dom] * 1e-3) / 1e9, 1)}

    # per-operation protocol on this workload, then host-call latency
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    print("bench: per-operation protocol", file=sys.stderr, flush=True)
    protocol = ops_report(measure_ops(torch, run, mg, mg0, args.reps, 3, flush), d) if args.reps > 0 else None
    host_us = host_call_latency(torch, mdg, run) if args.reps > 0 else None

    autograd = None
    if not args.no_autograd:
        mg.copy_(mg0)
        autograd = time_autograd(mdg, d, args.steps, max(args.warmup, 1), ms_per_step, flop_op)

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(d, args.cpu_seconds)

    # the other workloads, one at a time, per operation
    del run, d, x, w, g, offs, mg, mg0, y, dx
    torch.cuda.empty_cache()
    configs = {}
    names = [] if args.configs in ("", "none") or args.reps <= 0 else [c for c in args.configs.split(",") if c != args.workload]
    for name in names:
        print(f"bench: per-operation protocol on {name}", file=sys.stderr, flush=True)
        dc = make_inputs(name, seed=0, device=dev, tensors=("x", "w", "g", "main_grad"))
        rc = Runners(mdg, torch, dc)
        mgc = dc["main_grad"]
        mgc0 = mgc.clone()
        rep = ops_report(measure_ops(torch, rc, mgc, mgc0, args.reps, 2, flush), dc)
        c = CONFIGS[name]
        configs[name] = {"E": c.E, "K": c.K, "N": c.N, "sum_m": c.M,
                         "nonempty_experts": int((dc["sizes"] > 0).sum()), "ops": rep}
        del rc, dc, mgc, mgc0
        torch.cuda.empty_cache()

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
        "ops_protocol": {"what": f"each operation alone, 1 GiB L2/MALL flush before each of {args.reps} reps, "
                                 "median of HIP-event times; accumulate from a pristine main_grad each rep",
                         "ops": protocol},
        "host_call": host_us,
        "configs": configs,
        "cpu_baseline": cpu,
        "autograd": autograd,
        "rerun_bitwise": rerun_ok,
        "rerun_checks": rerun,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
