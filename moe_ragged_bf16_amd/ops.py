"""Python entry points over the C ABI, for torch tensors on a ROCm device.

Each function marshals pointers, sizes and the current HIP stream and calls the
library; every step of the computation runs in the gfx950 kernels.  torch
supplies device memory (outputs and the wgrad workspace) and the stream.

Signatures follow the one-shot functions of the Cake ragged BF16 grouped GEMM
API page and flashinfer PR #8924 ("Deterministic weight-gradient
accumulation"): grouped_det_gemm_fwd(x, w, offs), grouped_det_gemm_dgrad(g, w,
offs) and grouped_det_gemm_wgrad(g, x, offs, out=None, out_dtype=None,
num_groups=None, *, accumulate=False).  ``offs`` is the int32 device tensor of
cumulative end offsets ``[E]`` or the ``m_indptr [E + 1]`` form with a leading
zero (told apart by its length).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _capi

__all__ = ["grouped_det_gemm_fwd", "grouped_det_gemm_dgrad", "grouped_det_gemm_wgrad",
           "fwd_workspace_bytes", "dgrad_workspace_bytes", "wgrad_workspace_bytes",
           "wgrad_chunk_rows", "zero_pad_rows", "grouped_mm_bf16"]


def _stream_handle(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _offs_ptr(offs: torch.Tensor, E: int) -> int:
    """Pointer to the E cumulative end offsets (skips m_indptr's leading zero)."""
    if offs.dtype != torch.int32 or offs.dim() != 1 or offs.device.type != "cuda":
        raise TypeError("offs must be a 1-D int32 device tensor")
    if not offs.is_contiguous():
        raise ValueError("offs must be contiguous")
    if offs.numel() == E:
        return offs.data_ptr()
    if offs.numel() == E + 1:
        return offs.data_ptr() + 4
    raise ValueError(f"offs has {offs.numel()} entries; expected E={E} (offs) or E+1 (m_indptr)")


def _written(t: torch.Tensor) -> None:
    """Bumps the version counter of a caller's tensor the library wrote in
    place, as an in-place torch op would (inference tensors have none)."""
    if not t.is_inference():
        torch.autograd.graph.increment_version(t)


def _same_device(*ts):
    d = ts[0].device
    for t in ts[1:]:
        if t.device != d:
            raise ValueError("all tensors must be on the same device")


def fwd_workspace_bytes(m_rows: int, n: int, k: int, num_groups: int) -> int:
    return int(_capi.load_library().grouped_det_gemm_fwd_workspace_bytes(m_rows, n, k, num_groups))


def dgrad_workspace_bytes(m_rows: int, n: int, k: int, num_groups: int) -> int:
    return int(_capi.load_library().grouped_det_gemm_dgrad_workspace_bytes(m_rows, n, k, num_groups))


def _workspace(workspace: Optional[torch.Tensor], need: int, device) -> torch.Tensor:
    """The caller's workspace (checked) or a fresh one from torch's allocator."""
    if workspace is None:
        return torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 or \
            not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    if workspace.numel() < need:
        raise ValueError(f"workspace too small: {workspace.numel()} < {need} bytes")
    if workspace.device.type != "cuda":
        raise ValueError(f"workspace must be on a ROCm device, got {workspace.device}")
    return workspace


def grouped_det_gemm_fwd(x: torch.Tensor, w: torch.Tensor, offs: torch.Tensor,
                         out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y[s_e:t_e] = X[s_e:t_e] @ W[e]^T, bf16 [M, N].  Rows past offs[E-1] of a
    freshly allocated Y are left uninitialised.  `workspace` (uint8, at least
    fwd_workspace_bytes()) is allocated per call when not given."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w, "w", torch.bfloat16, 3)
    M, K = x.shape
    E, N, K2 = w.shape
    if K2 != K:
        raise ValueError(f"x has K={K} but w has K={K2}")
    given = out is not None
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must have shape {(M, N)}")
    _same_device(x, w, offs, out)
    op = _offs_ptr(offs, E)
    ws = _workspace(workspace, fwd_workspace_bytes(M, N, K, E), x.device)
    _same_device(x, ws)
    with torch.cuda.device(x.device):
        st = _capi.load_library().grouped_det_gemm_fwd(
            x.data_ptr(), w.data_ptr(), op, out.data_ptr(), M, N, K, E,
            ws.data_ptr(), ws.numel(), _stream_handle(x))
    _capi.check("grouped_det_gemm_fwd", st)
    if given:
        _written(out)
    return out


def grouped_det_gemm_dgrad(g: torch.Tensor, w: torch.Tensor, offs: torch.Tensor,
                           out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dX[s_e:t_e] = G[s_e:t_e] @ W[e], bf16 [M, K].  `workspace` (uint8, at
    least dgrad_workspace_bytes()) is allocated per call when not given."""
    _need(g, "g", torch.bfloat16, 2)
    _need(w, "w", torch.bfloat16, 3)
    M, N = g.shape
    E, N2, K = w.shape
    if N2 != N:
        raise ValueError(f"g has N={N} but w has N={N2}")
    given = out is not None
    if out is None:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=g.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, K):
        raise ValueError(f"out must have shape {(M, K)}")
    _same_device(g, w, offs, out)
    op = _offs_ptr(offs, E)
    ws = _workspace(workspace, dgrad_workspace_bytes(M, N, K, E), g.device)
    _same_device(g, ws)
    with torch.cuda.device(g.device):
        st = _capi.load_library().grouped_det_gemm_dgrad(
            g.data_ptr(), w.data_ptr(), op, out.data_ptr(), M, N, K, E,
            ws.data_ptr(), ws.numel(), _stream_handle(g))
    _capi.check("grouped_det_gemm_dgrad", st)
    if given:
        _written(out)
    return out


def wgrad_workspace_bytes(m_rows: int, n: int, k: int, num_groups: int) -> int:
    return int(_capi.load_library().grouped_det_gemm_wgrad_workspace_bytes(m_rows, n, k, num_groups))


def wgrad_chunk_rows(m_rows: int, n: int, k: int, num_groups: int) -> int:
    return int(_capi.load_library().grouped_det_gemm_wgrad_chunk_rows(m_rows, n, k, num_groups))


def grouped_det_gemm_wgrad(g: torch.Tensor, x: torch.Tensor, offs: torch.Tensor,
                           out: Optional[torch.Tensor] = None, out_dtype=None,
                           num_groups: Optional[int] = None, *, accumulate: bool = False,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dW[e] = G[s_e:t_e]^T @ X[s_e:t_e], [E, N, K] in bf16 or fp32.

    With ``accumulate=True`` the product is added into ``out`` with the bits
    of ``out.add_(dW)`` for this function's own overwrite dW in out's dtype:
    fp32, RN32(out + dW); bf16, RNE_bf16(RN32(out + RNE_bf16(dW))).  E comes
    from ``out``, else ``num_groups``, else the length of ``offs``.
    ``workspace`` (uint8 device tensor) is allocated when not given.
    """
    if not isinstance(accumulate, bool):
        raise TypeError("accumulate must be a bool")
    _need(g, "g", torch.bfloat16, 2)
    _need(x, "x", torch.bfloat16, 2)
    M, N = g.shape
    M2, K = x.shape
    if M2 != M:
        raise ValueError(f"g has {M} rows but x has {M2}")
    if out is not None:
        E = out.shape[0]
    elif num_groups is not None:
        E = int(num_groups)
    else:
        E = offs.numel()
    if out_dtype is not None and out is not None and out.dtype != out_dtype:
        raise TypeError("out_dtype must be None or equal to out.dtype")
    given = out is not None
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
    with torch.cuda.device(g.device):
        st = _capi.load_library().grouped_det_gemm_wgrad(
            g.data_ptr(), x.data_ptr(), op, out.data_ptr(), dt_code, int(accumulate),
            M, N, K, E, ws.data_ptr(), ws.numel(), _stream_handle(g))
    _capi.check("grouped_det_gemm_wgrad", st)
    if given:
        _written(out)
    return out


def zero_pad_rows(out: torch.Tensor, offs: torch.Tensor, num_groups: int) -> torch.Tensor:
    """Writes zeros over the rows of ``out`` [M, C] at or past offs[E-1] (rows
    that belong to no group), reading offs on the device only."""
    if not isinstance(out, torch.Tensor) or out.dim() != 2 or out.device.type != "cuda":
        raise ValueError("out must be a 2-D device tensor")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    E = int(num_groups)
    _same_device(out, offs)
    op = _offs_ptr(offs, E)
    row_bytes = out.shape[1] * out.element_size()
    with torch.cuda.device(out.device):
        st = _capi.load_library().grouped_det_gemm_zero_pad_rows(
            out.data_ptr(), op, out.shape[0], row_bytes, E, _stream_handle(out))
    _capi.check("grouped_det_gemm_zero_pad_rows", st)
    _written(out)
    return out


def grouped_mm_bf16(a: torch.Tensor, b: torch.Tensor, m_indptr: torch.Tensor,
                    out: Optional[torch.Tensor] = None, *, backend: str = "cake") -> torch.Tensor:
    """The stable grouped GEMM forward: ``out[m_indptr[e]:m_indptr[e+1]] =
    a[...] @ b[e]^T`` for a [cum_m, K], b [E, N, K] and m_indptr [E + 1] (int32,
    device, leading zero), bf16 out [cum_m, N] (Cake ragged BF16 grouped GEMM API
    page, "Stable API opt-in").  Rows past m_indptr[E] are zero.  The only
    backend is this library's (``backend="cake"``, the name the stable API uses
    for it); there is no tactic index."""
    if backend != "cake":
        raise ValueError(f"grouped_mm_bf16: unknown backend {backend!r} (only 'cake')")
    if not isinstance(m_indptr, torch.Tensor) or m_indptr.dim() != 1 or \
            not isinstance(b, torch.Tensor) or b.dim() != 3 or m_indptr.numel() != b.shape[0] + 1:
        raise ValueError("grouped_mm_bf16: m_indptr must be 1-D with E + 1 entries for b [E, N, K]")
    y = grouped_det_gemm_fwd(a, b, m_indptr, out=out)
    zero_pad_rows(y, m_indptr, b.shape[0])
    return y
