"""Plain, slow, obviously correct ragged grouped GEMM on the CPU (NumPy).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

bf16 data is handled as its raw 16-bit patterns (``numpy.uint16``).  Widening a
bf16 value to fp32 is exact (the bf16 pattern is the top half of the fp32
pattern), and fp32 widens exactly to fp64.  Products and sums are taken in fp64
(``precision="fp64"``, the default: the reference precision of the GPU test
description in flashinfer PR #8924, "Tests"), or in fp32 with ``precision="fp32"``
(the accumulation precision the API page states for the GPU programs).  A
library matmul (NumPy ``@``) serves as the per-group product; nothing is blocked,
fused or reordered beyond one product per group.
"""
from __future__ import annotations

import numpy as np

_PREC = {"fp64": np.float64, "fp32": np.float32}


# --------------------------------------------------------------------------
# bf16 <-> fp32
# --------------------------------------------------------------------------
def widen_bf16(bits) -> np.ndarray:
    """Exact bf16 -> fp32 widening: the 16 bits become the high half of fp32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16_rne(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even.

    Keeps the sign, exponent and top 7 mantissa bits.  The 16 dropped bits are
    compared with half an ulp (0x8000): above rounds up, below truncates, equal
    rounds to the even neighbour.  A carry out of the mantissa correctly bumps
    the exponent (up to infinity).  NaN stays NaN (quiet bit forced on so that the
    truncation cannot turn it into infinity).
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep = u >> np.uint64(16)
    low = u & np.uint64(0xFFFF)
    odd = keep & np.uint64(1)
    round_up = (low > 0x8000) | ((low == 0x8000) & (odd == 1))
    r = keep + round_up.astype(np.uint64)
    nan = np.isnan(f)
    r = np.where(nan, (keep | np.uint64(0x0040)), r)
    return (r & np.uint64(0xFFFF)).astype(np.uint16)


# --------------------------------------------------------------------------
# groups
# --------------------------------------------------------------------------
def offs_from_indptr(m_indptr) -> np.ndarray:
    """``m_indptr[E + 1]`` (leading zero) -> ``offs[E]`` (cumulative ends)."""
    ip = np.asarray(m_indptr, dtype=np.int64)
    if ip.ndim != 1 or ip.shape[0] < 1 or ip[0] != 0:
        raise ValueError("m_indptr must be 1-D with a leading zero")
    return ip[1:]


def group_ranges(offs, m_rows: int):
    """Row range [s_e, t_e) of every group from cumulative end offsets.

    Group e spans rows offs[e-1] .. offs[e]-1, with offs[-1] read as 0 (API page,
    operations table).  Offsets must be non-decreasing and within [0, m_rows];
    rows at or past offs[E-1] belong to no group.
    """
    o = np.asarray(offs, dtype=np.int64)
    if o.ndim != 1:
        raise ValueError("offs must be 1-D")
    ranges = []
    prev = 0
    for e in range(o.shape[0]):
        t = int(o[e])
        if t < prev or t > m_rows:
            raise ValueError(f"offs[{e}]={t} is not a valid cumulative end offset")
        ranges.append((prev, t))
        prev = t
    return ranges


# --------------------------------------------------------------------------
# the three operations
# --------------------------------------------------------------------------
def _f(bits, precision):
    return widen_bf16(bits).astype(_PREC[precision])


def fwd(x_bits, w_bits, offs, precision: str = "fp64") -> np.ndarray:
    """Y[s:t] = X[s:t] @ W[e].T for every group e (rows outside groups: NaN)."""
    M = x_bits.shape[0]
    E, N, K = w_bits.shape
    assert x_bits.shape == (M, K)
    y = np.full((M, N), np.nan, dtype=_PREC[precision])
    for e, (s, t) in enumerate(group_ranges(offs, M)):
        if t > s:
            y[s:t] = _f(x_bits[s:t], precision) @ _f(w_bits[e], precision).T
    return y


def dgrad(g_bits, w_bits, offs, precision: str = "fp64") -> np.ndarray:
    """dX[s:t] = G[s:t] @ W[e] for every group e (rows outside groups: NaN)."""
    M = g_bits.shape[0]
    E, N, K = w_bits.shape
    assert g_bits.shape == (M, N)
    dx = np.full((M, K), np.nan, dtype=_PREC[precision])
    for e, (s, t) in enumerate(group_ranges(offs, M)):
        if t > s:
            dx[s:t] = _f(g_bits[s:t], precision) @ _f(w_bits[e], precision)
    return dx


def wgrad(g_bits, x_bits, offs, precision: str = "fp64") -> np.ndarray:
    """dW[e] = G[s:t].T @ X[s:t]; exactly zero for an empty group."""
    M, N = g_bits.shape
    K = x_bits.shape[1]
    assert x_bits.shape[0] == M
    ranges = group_ranges(offs, M)
    dw = np.zeros((len(ranges), N, K), dtype=_PREC[precision])
    for e, (s, t) in enumerate(ranges):
        if t > s:
            dw[e] = _f(g_bits[s:t], precision).T @ _f(x_bits[s:t], precision)
    return dw


# Row- and expert-restricted forms for large workloads: the same definitions,
# evaluated only where a test samples.
def _expert_of_rows(offs, m_rows, rows):
    ranges = group_ranges(offs, m_rows)
    ends = np.array([t for _, t in ranges], dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    e = np.searchsorted(ends, rows, side="right")
    if np.any(e >= len(ranges)):
        raise ValueError("a sampled row belongs to no group")
    return e


def fwd_rows(x_bits, w_bits, offs, rows, precision: str = "fp64") -> np.ndarray:
    """Rows ``rows`` of Y: Y[i] = X[i] @ W[e(i)].T, e(i) the group holding row i."""
    M = x_bits.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    es = _expert_of_rows(offs, M, rows)
    out = np.empty((rows.shape[0], w_bits.shape[1]), dtype=_PREC[precision])
    for e in np.unique(es):
        sel = es == e
        out[sel] = _f(x_bits[rows[sel]], precision) @ _f(w_bits[e], precision).T
    return out


def dgrad_rows(g_bits, w_bits, offs, rows, precision: str = "fp64") -> np.ndarray:
    """Rows ``rows`` of dX: dX[i] = G[i] @ W[e(i)]."""
    M = g_bits.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    es = _expert_of_rows(offs, M, rows)
    out = np.empty((rows.shape[0], w_bits.shape[2]), dtype=_PREC[precision])
    for e in np.unique(es):
        sel = es == e
        out[sel] = _f(g_bits[rows[sel]], precision) @ _f(w_bits[e], precision)
    return out


def wgrad_expert(g_bits_e, x_bits_e, precision: str = "fp64") -> np.ndarray:
    """dW[e] from the rows of group e alone: G_e.T @ X_e (zeros if no rows)."""
    m, N = g_bits_e.shape
    K = x_bits_e.shape[1]
    if m == 0:
        return np.zeros((N, K), dtype=_PREC[precision])
    return _f(g_bits_e, precision).T @ _f(x_bits_e, precision)


# --------------------------------------------------------------------------
# accumulate (flashinfer PR #8924, "Design and numerics")
# --------------------------------------------------------------------------
def accumulate_fp32(out_f32, dw_f32) -> np.ndarray:
    """fp32 out: RN32(out + dW), one IEEE single-precision add per element."""
    a = np.asarray(out_f32, dtype=np.float32)
    b = np.asarray(dw_f32, dtype=np.float32)
    return np.add(a, b, dtype=np.float32)


def accumulate_bf16(out_bits, dw_bits) -> np.ndarray:
    """bf16 out: the bf16 dW is added in bf16.

    Reading taken: each element becomes RNE_bf16(RN32(f32(out) + f32(dW))), the
    way a framework adds two bf16 tensors (widen both exactly, one fp32 add,
    round the sum to bf16 with ties to even).
    """
    s = np.add(widen_bf16(out_bits), widen_bf16(dw_bits), dtype=np.float32)
    return round_bf16_rne(s)
