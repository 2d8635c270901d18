"""Autograd over the three entry points, with Megatron-style fused weight-gradient
accumulation.

``cake_grouped_det_mm(x, w, offs, *, fuse_wgrad_accumulation=False)`` computes
``Y = grouped_det_gemm_fwd(x, w, offs)``; its backward gives ``x.grad`` with the
dgrad kernel and the weight gradient with the wgrad kernel (Cake ragged BF16
grouped GEMM API page, "Autograd"; flashinfer PR #8924, "Fused weight-gradient
accumulation into main_grad").

Rows of ``x`` at or past ``offs[E-1]`` belong to no group: the forward writes
zeros into those rows of Y and the backward gives them a zero gradient (both
filled on the device, without reading offs on the host).

Without fusion the weight gradient is returned in w's dtype (bf16: the
overwrite wgrad rounded once) and autograd's AccumulateGrad adds it to
``w.grad``.  With ``fuse_wgrad_accumulation=True`` the backward instead adds the
deterministic dW into ``w.main_grad`` (fp32 or bf16) with the wgrad kernel's
accumulate epilogue, which gives the bits ``main_grad.add_(dW)`` would, dW being
the overwrite result in main_grad's dtype.  The Megatron / Transformer Engine
convention of that flag:

  * ``w.main_grad`` must be a tensor of w's shape and device, fp32 or bf16,
    with unit stride along K and no two elements sharing memory; it is checked
    when a forward is recorded by autograd and again, with its memory-sharing
    rules, at the backward, which reads the attribute anew (a main_grad
    re-pointed between the two is the one that receives the add);
  * if w has an attribute ``grad_added_to_main_grad``, the backward sets it to
    True and returns a fresh placeholder of w's shape and dtype for w's
    gradient (zeros when ``w.zero_out_wgrad`` is true, else uninitialised);
    otherwise it returns None for w;
  * every backward adds once: a graph backpropagated twice with
    ``retain_graph=True`` adds twice, and so does an ``autograd.grad`` whose
    inputs leave out w; a frozen w (``requires_grad=False``) gets nothing;
  * non-reentrant checkpoints, nested or not, work; a reentrant checkpoint
    records the forward only when it recomputes it, with a detached copy of w
    that has no ``main_grad``, and its backward raises ValueError.

In both modes ``create_graph=True`` raises NotImplementedError (the backward is
not differentiable), and so does ``torch.jit.trace``.  ``torch.compile`` with
``fullgraph=True`` fails at the same refusal; otherwise torch.compile runs the
call eagerly outside its graphs.

Memory: a non-contiguous (but valid) main_grad is accumulated through a
contiguous copy; the workspaces (fp32 partial tiles of experts split into row
chunks and of split tail units) are allocated per call from torch's caching
allocator.  Under ``torch.use_deterministic_algorithms(True)``
with ``fill_uninitialized_memory`` torch fills the fresh outputs and the
placeholder with NaN before the kernels write them (an extra pass over each);
the results are unchanged.
"""
from __future__ import annotations

import torch

from . import ops

__all__ = ["CakeGroupedDetMm", "cake_grouped_det_mm"]

_MAIN_GRAD_DTYPES = (torch.float32, torch.bfloat16)


def _byte_range(t: torch.Tensor):
    """[lo, hi) of the bytes a strided tensor can touch (empty for numel 0)."""
    if t.numel() == 0:
        return (0, 0)
    lo = t.data_ptr()
    span = 1 + sum((n - 1) * s for n, s in zip(t.shape, t.stride()))
    return (lo, lo + span * t.element_size())


def _shares_memory(a: torch.Tensor, b: torch.Tensor) -> bool:
    ra, rb = _byte_range(a), _byte_range(b)
    if ra[0] == ra[1] or rb[0] == rb[1]:
        return False
    return ra[0] < rb[1] and rb[0] < ra[1]


def _elements_overlap(t: torch.Tensor) -> bool:
    """True if two elements of t share memory (a stride-0 or interleaved view)."""
    dims = sorted((s, n) for n, s in zip(t.shape, t.stride()) if n > 1)
    span = 1  # elements covered by the dims taken so far
    for s, n in dims:
        if s < span:
            return True
        span = s * (n - 1) + span
    return False


def _main_grad(w: torch.Tensor, where: str) -> torch.Tensor:
    mg = getattr(w, "main_grad", None)
    if not isinstance(mg, torch.Tensor):
        raise ValueError(
            f"cake_grouped_det_mm(fuse_wgrad_accumulation=True) at the {where}: w has no main_grad tensor "
            "(a reentrant checkpoint passes a detached copy of w; use use_reentrant=False)")
    if mg.dtype not in _MAIN_GRAD_DTYPES:
        raise TypeError(f"w.main_grad must be float32 or bfloat16, got {mg.dtype}")
    if tuple(mg.shape) != tuple(w.shape):
        raise ValueError(f"w.main_grad has shape {tuple(mg.shape)}, w has {tuple(w.shape)}")
    if mg.device != w.device:
        raise ValueError(f"w.main_grad is on {mg.device}, w on {w.device}")
    if mg.numel() and mg.stride(-1) != 1 and mg.shape[-1] > 1:
        raise ValueError("w.main_grad must have unit stride along K (its last dimension)")
    if _elements_overlap(mg):
        raise ValueError("w.main_grad has overlapping rows or experts (an expanded or aliased view)")
    return mg


def _accumulate_into(main_grad: torch.Tensor, dy, x, offs) -> None:
    E = main_grad.shape[0]
    if main_grad.is_contiguous():
        ops.grouped_det_gemm_wgrad(dy, x, offs, out=main_grad, accumulate=True)
        return
    tmp = main_grad.contiguous()
    ops.grouped_det_gemm_wgrad(dy, x, offs, out=tmp, num_groups=E, accumulate=True)
    main_grad.copy_(tmp)


class CakeGroupedDetMm(torch.autograd.Function):
    """``Y = X @ W[e]^T`` per group, differentiable in X and W.

    ``apply(x, w, offs, _launch=None, fuse_wgrad_accumulation=False)``: the
    fourth argument is reserved and must be None (TypeError otherwise); the
    fifth must be a bool (ValueError otherwise).
    """

    @classmethod
    def apply(cls, x, w, offs, _launch=None, fuse_wgrad_accumulation=False):
        if _launch is not None:
            raise TypeError("CakeGroupedDetMm.apply: the fourth argument is reserved and must be None")
        if not isinstance(fuse_wgrad_accumulation, bool):
            raise ValueError("fuse_wgrad_accumulation must be a bool, got "
                             f"{type(fuse_wgrad_accumulation).__name__}")
        if torch.jit.is_tracing():
            raise NotImplementedError("cake_grouped_det_mm cannot be traced by torch.jit.trace")
        # A forward recorded during a backward pass is a checkpoint's
        # recomputation: its node is discarded (the backward that runs is the
        # original forward's), and it may see a detached copy of w.
        if fuse_wgrad_accumulation and torch.is_grad_enabled() and isinstance(w, torch.Tensor) \
                and w.requires_grad and torch._C._current_autograd_node() is None:
            _main_grad(w, "forward")
        return super().apply(x, w, offs, None, fuse_wgrad_accumulation)

    @staticmethod
    def forward(ctx, x, w, offs, _launch, fuse_wgrad_accumulation):
        y = ops.grouped_det_gemm_fwd(x, w, offs)
        ops.zero_pad_rows(y, offs, w.shape[0])
        ctx.save_for_backward(x, w, offs)
        ctx.fuse = fuse_wgrad_accumulation
        # The caller's w itself: the backward reads its main_grad and
        # grad_added_to_main_grad attributes (a checkpoint may hand back a
        # different tensor object for the saved w).
        ctx.w_obj = w if fuse_wgrad_accumulation else None
        return y

    @staticmethod
    def backward(ctx, dy):
        if torch.is_grad_enabled():
            raise NotImplementedError("cake_grouped_det_mm has no double backward (create_graph=True)")
        x, w, offs = ctx.saved_tensors
        dy = dy.contiguous()
        need_x, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        E = w.shape[0]
        dx = dw = None
        if ctx.fuse and need_w:
            w_obj = ctx.w_obj
            mg = _main_grad(w_obj, "backward")
            for name, t in (("the output gradient", dy), ("x", x), ("offs", offs), ("w", w)):
                if _shares_memory(mg, t):
                    raise ValueError(f"w.main_grad shares memory with {name}")
        if need_x:
            dx = ops.grouped_det_gemm_dgrad(dy, w, offs)
            ops.zero_pad_rows(dx, offs, E)
        if need_w:
            if ctx.fuse:
                _accumulate_into(mg, dy, x, offs)
                if hasattr(w_obj, "grad_added_to_main_grad"):
                    w_obj.grad_added_to_main_grad = True
                    if getattr(w_obj, "zero_out_wgrad", False):
                        dw = torch.zeros(w_obj.shape, dtype=w_obj.dtype, device=w_obj.device)
                    else:
                        dw = torch.empty(w_obj.shape, dtype=w_obj.dtype, device=w_obj.device)
            else:
                dw = ops.grouped_det_gemm_wgrad(dy, x, offs, out_dtype=w.dtype, num_groups=E)
        return dx, dw, None, None, None


def cake_grouped_det_mm(x: torch.Tensor, w: torch.Tensor, offs: torch.Tensor, *,
                        fuse_wgrad_accumulation: bool = False) -> torch.Tensor:
    """Differentiable ragged grouped GEMM ``Y[s_e:t_e] = X[s_e:t_e] @ W[e]^T``.

    x [M, K] bf16, w [E, N, K] bf16, offs int32 ``[E]`` (cumulative ends) or
    ``[E + 1]`` (m_indptr) on the device; returns Y [M, N] bf16 with zero rows
    past offs[E-1].  See the module docstring for the fused accumulation.
    """
    if torch.compiler.is_compiling():
        raise NotImplementedError("cake_grouped_det_mm cannot be compiled by torch.compile")
    return _apply_eagerly(x, w, offs, fuse_wgrad_accumulation)


@torch.compiler.disable
def _apply_eagerly(x, w, offs, fuse_wgrad_accumulation):
    # The library calls are opaque to torch.compile: when it does not stop at
    # the refusal above (it then runs the caller's frame without compiling it),
    # this call stays out of its graphs.
    return CakeGroupedDetMm.apply(x, w, offs, None, fuse_wgrad_accumulation)
