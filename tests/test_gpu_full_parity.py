"""Every output element at the full sizes of the four large workloads (seed 0)
against the CPU oracle: fwd, dgrad, wgrad fp32 and wgrad bf16, group by group.

The oracle runs here in fp32 (NumPy BLAS sgemm, one product per group: the plain
CPU fp32 per-group matmul the operations table defines), which finishes about
2 TFLOP per operation in seconds on the host cores; the fp64 form pins it in the
CPU tests.  Data moves one expert at a time, so host memory stays bounded
(an expert's W, its rows of X, G, Y, dX and its dW).  Gates as everywhere: per
group, max |gpu - ref| / max |ref| <= 2e-2 for bf16 outputs and 1e-3 for fp32
dW; empty groups exactly zero dW.
"""
import time

import numpy as np
import pytest
import torch

import moe_ragged_bf16_amd as mdg
import oracle
from workloads import make_inputs
from _parity import TOL_BF16, TOL_FP32, bits, ranges

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _f32(t):
    """GPU output -> float32 on the host (bf16 widened exactly)."""
    if t.dtype == torch.bfloat16:
        return oracle.widen_bf16(bits(t))
    return t.detach().cpu().numpy()


def _err(gpu, ref):
    """max |gpu - ref| / max |ref| in fp32 (a NaN or Inf in gpu makes it NaN or
    Inf, which fails every gate); 0 for an all-zero pair."""
    diff = float(np.max(np.abs(gpu - ref)))
    scale = float(np.max(np.abs(ref)))
    return diff / scale if scale > 0 else (0.0 if diff == 0 else float("inf"))


@pytest.mark.parametrize("name", ["mixtral", "fine", "skewed", "stress"])
def test_full_size_every_element(name):
    t0 = time.perf_counter()
    d = make_inputs(name, seed=0, device=DEV)
    E, N, K, M = d["E"], d["N"], d["K"], d["M"]
    print(f"{name}: every element, E={E} N={N} K={K} M={M}", flush=True)
    y = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    dx = mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"])
    dw32 = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)
    dw16 = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    worst = {"fwd": 0.0, "dgrad": 0.0, "wgrad fp32": 0.0, "wgrad bf16": 0.0}
    one = np.array([0], dtype=np.int32)
    for e, (s, t) in enumerate(ranges(d["sizes"])):
        m = t - s
        if m == 0:
            assert torch.all(dw32[e].view(torch.int32) == 0) and torch.all(dw16[e].view(torch.int16) == 0), e
            continue
        one[0] = m
        X, G, W = bits(d["x"][s:t]), bits(d["g"][s:t]), bits(d["w"][e:e + 1])
        checks = (("fwd", y[s:t], oracle.fwd(X, W, one, precision="fp32")),
                  ("dgrad", dx[s:t], oracle.dgrad(G, W, one, precision="fp32")))
        for op, got, ref in checks:
            worst[op] = max(worst[op], _err(_f32(got), ref))
        ref_dw = oracle.wgrad_expert(G, X, precision="fp32")
        worst["wgrad fp32"] = max(worst["wgrad fp32"], _err(_f32(dw32[e]), ref_dw))
        worst["wgrad bf16"] = max(worst["wgrad bf16"], _err(_f32(dw16[e]), ref_dw))
    print(f"  worst per-group error: " + ", ".join(f"{k} {v:.2e}" for k, v in worst.items())
          + f" ({time.perf_counter() - t0:.0f} s)", flush=True)
    assert all(np.isfinite(v) for v in worst.values()), worst
    assert worst["fwd"] <= TOL_BF16 and worst["dgrad"] <= TOL_BF16, worst
    assert worst["wgrad fp32"] <= TOL_FP32 and worst["wgrad bf16"] <= TOL_BF16, worst
