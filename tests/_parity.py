"""Helpers shared by the GPU parity tests: moving tensors to NumPy and the
tolerance metric.

Metric (the reading of "max relative error" used throughout): for each group,
err = max |gpu - ref| / max |ref| over that group's output block (its rows of
Y / dX, or its dW[e]).  Elementwise |a - b| / |b| is ill-posed near zero.  Any
NaN or Inf in a compared block fails.  Gates: 2e-2 for bf16 outputs and 1e-3
for fp32 wgrad.
"""
import numpy as np
import torch

import oracle

TOL_BF16 = 2e-2
TOL_FP32 = 1e-3


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> uint16 bit patterns on the host."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def values(t: torch.Tensor) -> np.ndarray:
    """GPU output -> float64 values on the host (bf16 widened exactly)."""
    if t.dtype == torch.bfloat16:
        return oracle.widen_bf16(bits(t)).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def block_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    if gpu.size == 0:
        return 0.0
    if not np.all(np.isfinite(gpu)):
        return float("inf")
    scale = np.max(np.abs(ref))
    diff = np.max(np.abs(gpu - ref))
    if scale == 0:
        return 0.0 if diff == 0 else float("inf")
    return float(diff / scale)


def group_errs(gpu: np.ndarray, ref: np.ndarray, sizes) -> list:
    """Per-group errors over consecutive row blocks of sizes[e] rows."""
    out = []
    s = 0
    for m in sizes:
        m = int(m)
        out.append(block_err(gpu[s:s + m], ref[s:s + m]))
        s += m
    return out


def ranges(sizes):
    s = 0
    res = []
    for m in sizes:
        res.append((s, s + int(m)))
        s += int(m)
    return res
