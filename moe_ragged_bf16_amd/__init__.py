"""Deterministic ragged BF16 grouped GEMM for MoE expert projections on MI355X.

fwd ``Y[g] = X[g] @ W[e]^T``, dgrad ``dX[g] = G[g] @ W[e]`` and wgrad
``dW[e] = G[g]^T @ X[g]`` over consecutive row groups given by device offsets,
with fp32 accumulation in a fixed order (bitwise reproducible, no atomics),
exactly-zero dW for empty groups and an optional fp32 accumulate into a
main_grad.  The computation is hand-written HIP for gfx950 behind the C ABI in
``include/moe_ragged_bf16.h``; this package is its thin torch binding.
"""
from ._capi import MdgError, load_library, status_string, EXPORTED  # noqa: F401
from .ops import (  # noqa: F401
    grouped_det_gemm_fwd,
    grouped_det_gemm_dgrad,
    grouped_det_gemm_wgrad,
    fwd_workspace_bytes,
    dgrad_workspace_bytes,
    wgrad_workspace_bytes,
    wgrad_chunk_rows,
)
from .ops import zero_pad_rows, grouped_mm_bf16  # noqa: F401
from .autograd import CakeGroupedDetMm, cake_grouped_det_mm  # noqa: F401
from .launch import (  # noqa: F401
    ACCUMULATE_MODES,
    GroupedDetGemmLaunch,
    prepare_grouped_det_gemm_fwd,
    prepare_grouped_det_gemm_dgrad,
    prepare_grouped_det_gemm_wgrad,
)
