"""Prepared launches: validate and bind once, launch many times.

``prepare_grouped_det_gemm_{fwd,dgrad,wgrad}`` take the arguments of the
one-shot functions of the same names, run all of their checks, allocate the
output (unless given) and the workspace (unless given) once, and return a
:class:`GroupedDetGemmLaunch` (Cake ragged BF16 grouped GEMM API page,
"Prepared launches"; flashinfer PR #8924, "API").  Its ``launch()`` enqueues the
bound kernels on the current stream with no allocation, no host
synchronisation and no memset, so it can be captured into a CUDA/HIP graph
(``torch.cuda.graph``).  The kernels read offs and the data on the device at
the time they run: offsets or values written in place into the bound tensors
between launches or graph replays are picked up.

Every ``launch()`` and every replay of a graph holding one computes again; an
accumulating wgrad launch adds again.  ``launch()`` (also while being captured)
bumps the output's version counter like an in-place torch op; a graph replay
runs no Python and does not.  The launch object keeps the bound tensors alive;
keep it (or them) alive while a graph that captured it may replay.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _capi
from .ops import (_need, _offs_ptr, _same_device, _stream_handle, _workspace, _written,
                  dgrad_workspace_bytes, fwd_workspace_bytes, wgrad_workspace_bytes)

__all__ = ["GroupedDetGemmLaunch", "prepare_grouped_det_gemm_fwd", "prepare_grouped_det_gemm_dgrad",
           "prepare_grouped_det_gemm_wgrad", "ACCUMULATE_MODES"]

# plan["accumulate"]: "fused" adds dW into the output in the wgrad epilogue
ACCUMULATE_MODES = ("off", "fused")
_OPS = ("fwd", "dgrad", "wgrad")


class GroupedDetGemmLaunch:
    """One prepared fwd, dgrad or wgrad launch over bound tensors."""

    def __init__(self, entry: str, handle: ctypes.c_void_p, out: torch.Tensor, bound: tuple):
        self._lib = _capi.load_library()
        self._h = handle
        self._entry = entry
        self.out = out
        self._bound = bound  # keeps the inputs, offs and workspace alive
        self.device = out.device
        info = _capi.LaunchInfo()
        _capi.check("grouped_det_gemm_launch_info",
                    self._lib.grouped_det_gemm_launch_info(self._h, ctypes.byref(info)))
        op = _OPS[info.op]
        self.plan = {
            "op": op,
            "kernels": int(info.kernels),
            "gemm_grid": int(info.gemm_grid),
            "workspace_bytes": int(info.workspace_bytes),
            "accumulate": ACCUMULATE_MODES[int(info.accumulate)],
            "out_dtype": out.dtype,
            "chunk_rows": int(info.chunk_rows) if op == "wgrad" else None,
            "tail_slots": int(info.tail_slots) if op != "wgrad" else None,
        }

    def launch(self) -> torch.Tensor:
        """Enqueue the bound kernels on the current stream; returns the output."""
        if self._h is None:
            raise RuntimeError(f"{self._entry}: launch used after close()")
        if torch.cuda.current_device() != self.device.index:
            with torch.cuda.device(self.device):
                st = self._lib.grouped_det_gemm_launch(self._h, _stream_handle(self.out))
        else:
            st = self._lib.grouped_det_gemm_launch(self._h, _stream_handle(self.out))
        _capi.check("grouped_det_gemm_launch", st)
        _written(self.out)
        return self.out

    def close(self) -> None:
        """Release the host-side launch object (enqueued work is unaffected)."""
        if self._h is not None:
            self._lib.grouped_det_gemm_launch_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass

    def __repr__(self):
        return f"GroupedDetGemmLaunch({self.plan})"


def _prepare(entry: str, fn, args, out, bound) -> GroupedDetGemmLaunch:
    h = ctypes.c_void_p()
    with torch.cuda.device(out.device):
        st = fn(*args, ctypes.byref(h))
    _capi.check(entry, st)
    return GroupedDetGemmLaunch(entry, h, out, bound)


def prepare_grouped_det_gemm_fwd(x: torch.Tensor, w: torch.Tensor, offs: torch.Tensor,
                                 out: Optional[torch.Tensor] = None,
                                 workspace: Optional[torch.Tensor] = None) -> GroupedDetGemmLaunch:
    """Prepared ``Y[s_e:t_e] = X[s_e:t_e] @ W[e]^T`` (bf16 [M, N])."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w, "w", torch.bfloat16, 3)
    M, K = x.shape
    E, N, K2 = w.shape
    if K2 != K:
        raise ValueError(f"x has K={K} but w has K={K2}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must have shape {(M, N)}")
    _same_device(x, w, offs, out)
    op = _offs_ptr(offs, E)
    ws = _workspace(workspace, fwd_workspace_bytes(M, N, K, E), x.device)
    _same_device(x, ws)
    lib = _capi.load_library()
    return _prepare("grouped_det_gemm_prepare_fwd", lib.grouped_det_gemm_prepare_fwd,
                    (x.data_ptr(), w.data_ptr(), op, out.data_ptr(), M, N, K, E, ws.data_ptr(), ws.numel()),
                    out, (x, w, offs, ws))


def prepare_grouped_det_gemm_dgrad(g: torch.Tensor, w: torch.Tensor, offs: torch.Tensor,
                                   out: Optional[torch.Tensor] = None,
                                   workspace: Optional[torch.Tensor] = None) -> GroupedDetGemmLaunch:
    """Prepared ``dX[s_e:t_e] = G[s_e:t_e] @ W[e]`` (bf16 [M, K])."""
    _need(g, "g", torch.bfloat16, 2)
    _need(w, "w", torch.bfloat16, 3)
    M, N = g.shape
    E, N2, K = w.shape
    if N2 != N:
        raise ValueError(f"g has N={N} but w has N={N2}")
    if out is None:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=g.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, K):
        raise ValueError(f"out must have shape {(M, K)}")
    _same_device(g, w, offs, out)
    op = _offs_ptr(offs, E)
    ws = _workspace(workspace, dgrad_workspace_bytes(M, N, K, E), g.device)
    _same_device(g, ws)
    lib = _capi.load_library()
    return _prepare("grouped_det_gemm_prepare_dgrad", lib.grouped_det_gemm_prepare_dgrad,
                    (g.data_ptr(), w.data_ptr(), op, out.data_ptr(), M, N, K, E, ws.data_ptr(), ws.numel()),
                    out, (g, w, offs, ws))


def prepare_grouped_det_gemm_wgrad(g: torch.Tensor, x: torch.Tensor, offs: torch.Tensor,
                                   out: Optional[torch.Tensor] = None, out_dtype=None,
                                   num_groups: Optional[int] = None, *, accumulate: bool = False,
                                   workspace: Optional[torch.Tensor] = None) -> GroupedDetGemmLaunch:
    """Prepared ``dW[e] = G[s_e:t_e]^T @ X[s_e:t_e]`` ([E, N, K], bf16 or fp32),
    or with ``accumulate=True`` its add into ``out`` (every launch adds)."""
    if not isinstance(accumulate, bool):
        raise TypeError("accumulate must be a bool")
    _need(g, "g", torch.bfloat16, 2)
    _need(x, "x", torch.bfloat16, 2)
    M, N = g.shape
    M2, K = x.shape
    if M2 != M:
        raise ValueError(f"g has {M} rows but x has {M2}")
    E = out.shape[0] if out is not None else (int(num_groups) if num_groups is not None else offs.numel())
    if out_dtype is not None and out is not None and out.dtype != out_dtype:
        raise TypeError("out_dtype must be None or equal to out.dtype")
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs out")
        dt = torch.bfloat16 if out_dtype is None else out_dtype
        if dt not in (torch.bfloat16, torch.float32):
            raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
        out = torch.empty((E, N, K), dtype=dt, device=g.device)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    _need(out, "out", out.dtype, 3)
    if tuple(out.shape) != (E, N, K):
        raise ValueError(f"out must have shape {(E, N, K)}")
    _same_device(g, x, offs, out)
    op = _offs_ptr(offs, E)
    ws = _workspace(workspace, wgrad_workspace_bytes(M, N, K, E), g.device)
    _same_device(g, ws)
    dt_code = _capi.MDG_FP32 if out.dtype == torch.float32 else _capi.MDG_BF16
    lib = _capi.load_library()
    return _prepare("grouped_det_gemm_prepare_wgrad", lib.grouped_det_gemm_prepare_wgrad,
                    (g.data_ptr(), x.data_ptr(), op, out.data_ptr(), dt_code, int(accumulate), M, N, K, E,
                     ws.data_ptr(), ws.numel()),
                    out, (g, x, offs, ws))
