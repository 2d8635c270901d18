"""Special input values on the GPU.

* NaN and Inf propagate as IEEE arithmetic says, to exactly the outputs that
  depend on them, and never into another group: a NaN in X[r, k] makes row r of
  Y NaN and column k of its expert's dW NaN; a NaN in G[r, n] makes row r of dX
  and row n of dW NaN; +Inf in X[r, k] makes Y[r, n] carry the sign of
  W[e][n, k]; +Inf in W[e][n, k] makes column n of the group's Y rows carry the
  sign of X[r, k] and column k of its dX rows the sign of G[r, n].  The expected
  masks are written out here from those rules (a BLAS product is not used for
  them: BLAS kernels may skip zero multiplicands, which changes NaN propagation).
  The layout has the fwd/dgrad tail split, a wgrad expert split into row chunks,
  a short wgrad unit (a group of at most 96 rows), an empty group, partial tiles
  in N and K and padding rows.
* Subnormal bf16 inputs are used as they are (not flushed to zero): products of
  subnormals and 2^64 match the oracle.
"""
import numpy as np
import pytest
import torch

import moe_ragged_bf16_amd as mdg
import oracle
from workloads import make_inputs
from _parity import TOL_BF16, TOL_FP32, bits, block_err, group_errs, ranges, values
from _plan import tail_plan

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SIZES = [100, 300, 50, 0, 200]
N, K, PAD = 264, 136, 7


def _layout_is_covered(M):
    assert tail_plan("fwd", SIZES, N, K, M=M)[2] >= 2 and tail_plan("dgrad", SIZES, N, K, M=M)[2] >= 2
    assert max(SIZES) > mdg.wgrad_chunk_rows(M, N, K, len(SIZES))      # a split expert
    assert any(0 < m <= 96 for m in SIZES)                               # a short wgrad unit


def test_nan_and_inf_stay_where_they_belong():
    d = make_inputs(sizes=SIZES, N=N, K=K, extra_rows=PAD, seed=31, device=DEV)
    M = d["M"]
    _layout_is_covered(M)
    starts = np.concatenate([[0], np.cumsum(SIZES)])
    # (row, column) of each planted value; groups: 1 (split), 2 (short), 0 (ring), 4
    x_nan = [(int(starts[1]) + 290, 5), (int(starts[2]) + 7, 130)]
    g_nan = [(int(starts[1]) + 3, 9), (int(starts[4]) + 150, 263)]
    x_inf = (int(starts[0]) + 40, 17)            # +Inf in X, group 0
    w_inf = (4, 200, 70)                         # +Inf in W[4][200, 70]
    for r, c in x_nan:
        d["x"][r, c] = float("nan")
    for r, c in g_nan:
        d["g"][r, c] = float("nan")
    d["x"][x_inf] = float("inf")
    d["w"][w_inf] = float("inf")
    X = oracle.widen_bf16(bits(d["x"])).astype(np.float64)
    G = oracle.widen_bf16(bits(d["g"])).astype(np.float64)
    W = oracle.widen_bf16(bits(d["w"])).astype(np.float64)
    print(f"special values: sizes={SIZES} N={N} K={K} pad={PAD}", flush=True)

    t = int(starts[-1])
    # (rows past the last group are never written: only the group rows are read back)
    y = values(mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])[:t])
    dx = values(mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"])[:t])
    dw = values(mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32))
    group_of = np.repeat(np.arange(len(SIZES)), SIZES)

    # expected fwd: NaN rows from x_nan; row x_inf: sign of W[e][:, k]; the group of
    # w_inf: column n gets the sign of X[r, k] on its rows
    ey_nan = np.zeros((t, N), bool)
    ey_inf = np.zeros((t, N), np.int8)
    for r, c in x_nan:
        ey_nan[r, :] = True
    r, c = x_inf
    ey_inf[r, :] = np.sign(W[group_of[r], :, c]).astype(np.int8)
    e, n, k = w_inf
    for r in range(int(starts[e]), int(starts[e + 1])):
        ey_inf[r, n] = np.sign(X[r, k])
    assert np.all(W[group_of[x_inf[0]], :, x_inf[1]] != 0) and np.all(X[starts[e]:starts[e + 1], k] != 0)
    assert np.array_equal(np.isnan(y[:t]), ey_nan)
    assert np.array_equal(np.where(np.isinf(y[:t]), np.sign(y[:t]), 0).astype(np.int8), ey_inf)

    # expected dgrad: NaN rows from g_nan; the group of w_inf: column k gets the sign of G[r, n]
    edx_nan = np.zeros((t, K), bool)
    edx_inf = np.zeros((t, K), np.int8)
    for r, c in g_nan:
        edx_nan[r, :] = True
    for r in range(int(starts[e]), int(starts[e + 1])):
        if not edx_nan[r, 0]:
            edx_inf[r, k] = np.sign(G[r, n])
    assert np.all(G[starts[e]:starts[e + 1], n][~edx_nan[starts[e]:starts[e + 1], 0]] != 0)
    assert np.array_equal(np.isnan(dx[:t]), edx_nan)
    assert np.array_equal(np.where(np.isinf(dx[:t]), np.sign(dx[:t]), 0).astype(np.int8), edx_inf)

    # expected wgrad: a NaN in X[r, c] -> column c of dW[e]; in G[r, c] -> row c of dW[e];
    # +Inf in X[r, c] -> column c of dW[e] with the sign of G[r, :] (no NaN in that row)
    edw_nan = np.zeros(dw.shape, bool)
    edw_inf = np.zeros(dw.shape, np.int8)
    for r, c in x_nan:
        edw_nan[group_of[r], :, c] = True
    for r, c in g_nan:
        edw_nan[group_of[r], c, :] = True
    r, c = x_inf
    edw_inf[group_of[r], :, c] = np.sign(G[r, :]).astype(np.int8)
    edw_inf[edw_nan] = 0
    assert np.all(G[r, :] != 0)
    assert np.array_equal(np.isnan(dw), edw_nan)
    assert np.array_equal(np.where(np.isinf(dw), np.sign(dw), 0).astype(np.int8), edw_inf)

    # everything else: finite and within the usual gates of the oracle on the same
    # inputs with the planted entries set to zero
    for r, c in x_nan + [x_inf]:
        X[r, c] = 0.0
    for r, c in g_nan:
        G[r, c] = 0.0
    W[w_inf] = 0.0
    xb = oracle.round_bf16_rne(X)
    gb = oracle.round_bf16_rne(G)
    wb = oracle.round_bf16_rne(W)
    offs = d["offs"].cpu().numpy()
    ry, rdx, rdw = oracle.fwd(xb, wb, offs), oracle.dgrad(gb, wb, offs), oracle.wgrad(gb, xb, offs)
    fy = ~(ey_nan | (ey_inf != 0))
    fdx = ~(edx_nan | (edx_inf != 0))
    fdw = ~(edw_nan | (edw_inf != 0))
    assert np.all(np.isfinite(y[:t][fy])) and np.all(np.isfinite(dx[:t][fdx])) and np.all(np.isfinite(dw[fdw]))
    assert max(group_errs(np.where(fy, y[:t], 0), np.where(fy, ry[:t], 0), SIZES)) <= TOL_BF16
    assert max(group_errs(np.where(fdx, dx[:t], 0), np.where(fdx, rdx[:t], 0), SIZES)) <= TOL_BF16
    assert max(block_err(np.where(fdw[e], dw[e], 0), np.where(fdw[e], rdw[e], 0)) for e in range(len(SIZES))) <= TOL_FP32


def test_subnormal_inputs_are_not_flushed():
    M, n, k = 48, 24, 72
    xb = np.full((M, k), 0x0001, dtype=np.uint16)      # 2^-133, the smallest subnormal bf16
    xb[:, 1::2] = 0x007F                               # the largest subnormal
    xb[1::2, :] |= 0x8000                              # and negative ones
    big = np.full((1, n, k), 0x5F80, dtype=np.uint16)  # 2^64
    gb = np.full((M, n), 0x5F80, dtype=np.uint16)

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)

    offs = torch.tensor([M], dtype=torch.int32, device=DEV)
    o = np.array([M], dtype=np.int32)
    xpos = xb & 0x7FFF                                 # wgrad sums over rows: all positive there
    y = values(mdg.grouped_det_gemm_fwd(dev(xb), dev(big), offs))
    dw = values(mdg.grouped_det_gemm_wgrad(dev(gb), dev(xpos), offs, out_dtype=torch.float32))
    ry = oracle.fwd(xb, big, o)
    rdw = oracle.wgrad(gb, xpos, o)
    assert np.all(ry != 0) and np.all(rdw != 0)
    assert np.all(y != 0) and np.all(dw != 0)
    assert max(group_errs(y, ry, [M])) <= TOL_BF16
    assert block_err(dw[0], rdw[0]) <= TOL_FP32
    # dgrad: subnormal W columns against 2^64 rows of G
    wsub = np.full((1, n, k), 0x0005, dtype=np.uint16)
    dx = values(mdg.grouped_det_gemm_dgrad(dev(gb), dev(wsub), offs))
    rdx = oracle.dgrad(gb, wsub, o)
    assert np.all(rdx != 0) and np.all(dx != 0)
    assert max(group_errs(dx, rdx, [M])) <= TOL_BF16
