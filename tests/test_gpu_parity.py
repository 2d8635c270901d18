"""GPU parity: the HIP path against the CPU oracle (fp64), element by element
on small ragged cases and on sampled outputs at the full workload sizes."""
import numpy as np
import pytest
import torch

import moe_ragged_bf16_amd as mdg
import oracle
from workloads import make_inputs
from _parity import TOL_BF16, TOL_FP32, bits, block_err, group_errs, values, ranges

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENTINEL = 0x7FC1   # a NaN pattern: rows outside every group must keep it


def _poisoned(shape, dtype):
    if dtype == torch.bfloat16:
        return torch.full(shape, SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    return torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)


def _run_all(d, wgrad_dtypes=(torch.bfloat16, torch.float32)):
    M, N, K, E = d["M"], d["N"], d["K"], d["E"]
    y = _poisoned((M, N), torch.bfloat16)
    dx = _poisoned((M, K), torch.bfloat16)
    mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"], out=y)
    mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"], out=dx)
    dws = {}
    for dt in wgrad_dtypes:
        dws[dt] = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out=_poisoned((E, N, K), dt))
    torch.cuda.synchronize()
    return y, dx, dws


def _check_full(d, label):
    """Every output element against the fp64 oracle."""
    y, dx, dws = _run_all(d)
    X, W, G = bits(d["x"]), bits(d["w"]), bits(d["g"])
    offs = d["offs"].cpu().numpy()
    sizes = d["sizes"]
    Mg = int(sizes.sum())
    ry = oracle.fwd(X, W, offs)
    rdx = oracle.dgrad(G, W, offs)
    rdw = oracle.wgrad(G, X, offs)
    ey = group_errs(values(y[:Mg]), ry[:Mg], sizes)
    edx = group_errs(values(dx[:Mg]), rdx[:Mg], sizes)
    assert max(ey, default=0) <= TOL_BF16, (label, "fwd", ey)
    assert max(edx, default=0) <= TOL_BF16, (label, "dgrad", edx)
    # rows past offs[E-1] are untouched
    if Mg < d["M"]:
        assert np.all(bits(y)[Mg:] == SENTINEL) and np.all(bits(dx)[Mg:] == SENTINEL), label
    for dt, tol in ((torch.bfloat16, TOL_BF16), (torch.float32, TOL_FP32)):
        dw = values(dws[dt])
        errs = [block_err(dw[e], rdw[e]) for e in range(d["E"])]
        assert max(errs) <= tol, (label, "wgrad", dt, errs)
        raw = dws[dt].cpu().view(torch.int16 if dt == torch.bfloat16 else torch.int32)
        for e, m in enumerate(sizes):
            if m == 0:
                assert torch.all(raw[e] == 0), (label, "empty expert must be +0.0", e)
    # bf16 dW is the RNE rounding of the fp32 dW (one shared reduction)
    assert torch.equal(dws[torch.float32].to(torch.bfloat16).view(torch.int16),
                       dws[torch.bfloat16].view(torch.int16)), label


def test_tiny_full():
    d = make_inputs("tiny", seed=0, device=DEV)
    _check_full(d, "tiny")


def test_tiny_indptr_form():
    d = make_inputs("tiny", seed=0, device=DEV)
    y1 = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    y2 = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["m_indptr"])
    dx1 = mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"])
    dx2 = mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["m_indptr"])
    w1 = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)
    w2 = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["m_indptr"], out_dtype=torch.float32, num_groups=4)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(dx1.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(w1.view(torch.int32), w2.view(torch.int32))


@pytest.mark.parametrize("sizes,N,K,pad", [
    ([1], 256, 64, 0),                       # one row, one reduction step
    ([0, 257, 0, 255, 256], 512, 320, 0),    # empties, tile +-1, k not a multiple of 256
    ([300, 1, 2, 63, 64, 65], 256, 192, 5),  # row padding past the last group
    ([0, 0, 0], 256, 128, 7),                # every group empty
    ([0, 0, 0, 0], 896, 576, 0),             # no rows at all (M = 0)
    ([1000, 3000], 256, 256, 0),             # long groups: wgrad row split
    ([700], 768, 576, 0),                    # one group, several tiles in N and K
    ([0, 257, 0, 255, 256], 320, 320, 2),    # n not a multiple of 256: partial last tile in n
    ([700, 3], 64, 64, 1),                   # n = 64: a single partial tile
    ([1000, 3000], 1088, 256, 0),            # partial n tile with the wgrad row split
    ([513, 0, 1, 1400], 2880, 2880, 3),      # n = k = 2880 (11.25 tiles of 256)
    # n and k multiples of 8 only: partial tiles 8 wide, and the last 32-deep
    # reduction stage of fwd (over k) or dgrad (over n) holds 8, 16 or 24 columns
    ([1, 300, 0, 40], 8, 8, 2),              # one stage of 8 columns, one partial tile
    ([257, 0, 513], 56, 200, 1),             # dgrad stage of 24, fwd stage of 8 (fwd split)
    ([0, 700, 33, 256], 264, 1032, 0),       # tiles of 8 in n and k; both splits end partial
    ([1000, 3000], 48, 120, 0),              # wgrad row split; stages of 16 and 24
    ([513, 0, 1, 1400], 2888, 80, 3),        # fwd stage of 16; dgrad split, last stage of 8
])
def test_small_ragged_full(sizes, N, K, pad):
    d = make_inputs(sizes=sizes, N=N, K=K, extra_rows=pad, seed=3, device=DEV)
    _check_full(d, f"sizes={sizes} N={N} K={K} pad={pad}")


def test_wgrad_split_is_exercised():
    # the cases above cover both a split (long groups) and no split
    assert mdg.wgrad_chunk_rows(4000, 256, 256, 2) < 3000
    assert mdg.wgrad_chunk_rows(512, 256, 256, 4) < 311


# ---------------------------------------------------------------- full sizes
def _sample_rows(sizes, per_group, rng):
    rows = []
    for s, t in ranges(sizes):
        if t == s:
            continue
        pick = {s, t - 1, min(t - 1, s + 255), min(t - 1, s + 256)}
        pick |= set(rng.integers(s, t, per_group).tolist())
        rows.extend(sorted(pick))
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("name", ["mixtral", "fine", "skewed", "stress", "gate_up_e32", "down_e4"])
def test_full_size_sampled(name):
    d = make_inputs(name, seed=0, device=DEV)
    rng = np.random.default_rng(1)
    y = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    dx = mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"])
    dw = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    sizes = d["sizes"]
    offs = d["offs"].cpu().numpy()
    rows = _sample_rows(sizes, 6, rng)
    rows_t = torch.from_numpy(rows).to(DEV)
    X = bits(d["x"][rows_t])
    G = bits(d["g"][rows_t])
    W = bits(d["w"])
    # sampled rows keep their group: build a compact offs over the sample
    owner = np.searchsorted(offs, rows, side="right")
    sub_sizes = np.bincount(owner, minlength=d["E"])
    sub_offs = np.cumsum(sub_sizes).astype(np.int32)
    ry = oracle.fwd(X, W, sub_offs)
    rdx = oracle.dgrad(G, W, sub_offs)
    gy, gdx = values(y[rows_t]), values(dx[rows_t])
    assert max(group_errs(gy, ry, sub_sizes)) <= TOL_BF16
    assert max(group_errs(gdx, rdx, sub_sizes)) <= TOL_BF16
    # wgrad: sampled dW rows (n) of every non-empty expert, plus empty experts
    n_pick = np.unique(np.concatenate([[0, d["N"] - 1], rng.integers(0, d["N"], 6)]))
    for e, (s, t) in enumerate(ranges(sizes)):
        got = dw[e][torch.from_numpy(n_pick).to(DEV)]
        if t == s:
            assert torch.all(got.view(torch.int32) == 0)
            continue
        Ge = bits(d["g"][s:t][:, torch.from_numpy(n_pick).to(DEV)].contiguous())
        Xe = bits(d["x"][s:t])
        ref = oracle.wgrad_expert(Ge, Xe)
        assert block_err(values(got), ref) <= TOL_FP32, (name, e)


def test_stable_grouped_mm_bf16():
    d = make_inputs(sizes=[0, 700, 1, 300, 257], N=512, K=320, extra_rows=4, seed=31, device=DEV)
    t = 1258
    y = mdg.grouped_mm_bf16(d["x"], d["w"], d["m_indptr"])
    ref = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    torch.cuda.synchronize()
    assert torch.equal(y[:t].view(torch.int16), ref[:t].view(torch.int16))
    assert torch.all(y[t:].view(torch.int16) == 0)
    with pytest.raises(ValueError):
        mdg.grouped_mm_bf16(d["x"], d["w"], d["offs"])            # the stable API takes m_indptr
    with pytest.raises(ValueError):
        mdg.grouped_mm_bf16(d["x"], d["w"], d["m_indptr"], backend="cudnn")


@pytest.mark.parametrize("name", ["mixtral", "stress"])
def test_adjoint_identity_full_size(name):
    """<Y, G> = <X, dX> = sum_e <W[e], dW[e]> over the group rows: all three equal
    sum_e <G_e^T X_e, W[e]>.  Computed in fp64 on the device from the three
    kernels' outputs at the full workload size; Y and dX are bf16-rounded, so the
    sides agree to about the bf16 rounding (a wrong index, sign or group in any one
    kernel breaks the equality by O(1))."""
    d = make_inputs(name, seed=0, device=DEV)
    print(f"adjoint identity: {name}", flush=True)
    t = int(d["sizes"].sum())
    y = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    dx = mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"])
    dw = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)
    pyg = y[:t].double() * d["g"][:t].double()
    pxdx = d["x"][:t].double() * dx[:t].double()
    yg, xdx = torch.sum(pyg).item(), torch.sum(pxdx).item()
    wdw = sum(torch.sum(d["w"][e].double() * dw[e].double()).item() for e in range(d["E"]))
    # the bf16 rounding of Y (resp. dX) perturbs each product by ~2^-9 of itself with
    # random sign: the sums then differ by ~2^-9 * ||products||_2 (the signed sums
    # themselves are of that norm's order, so an error in any kernel shows as O(1))
    ny, nx = torch.linalg.vector_norm(pyg).item(), torch.linalg.vector_norm(pxdx).item()
    print(f"  <Y,G>={yg:.6g} <X,dX>={xdx:.6g} sum<W,dW>={wdw:.6g} "
          f"|dy|/||YG||={abs(yg - wdw) / ny:.2e} |dx|/||XdX||={abs(xdx - wdw) / nx:.2e}", flush=True)
    assert abs(yg - wdw) <= 1e-2 * ny, (name, yg, wdw, ny)
    assert abs(xdx - wdw) <= 1e-2 * nx, (name, xdx, wdw, nx)
    assert abs(wdw) > 0.05 * ny, (name, wdw, ny)      # the identity is not vacuous here


def test_single_group_equals_dense():
    """E = 1: the grouped ops are plain dense products (fp32 torch matmul as the
    reference, within the bf16 output tolerance)."""
    d = make_inputs(sizes=[1000], N=512, K=320, seed=41, device=DEV)
    x, w, g = d["x"].float(), d["w"][0].float(), d["g"].float()
    y = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"]).float()
    dx = mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"]).float()
    dw = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)[0]
    for got, ref, tol in ((y, x @ w.T, TOL_BF16), (dx, g @ w, TOL_BF16), (dw, g.T @ x, TOL_FP32)):
        err = ((got - ref).abs().max() / ref.abs().max()).item()
        assert err <= tol, err


@pytest.mark.parametrize("E", [1024, 1000])
def test_max_group_count(E):
    """The largest supported number of groups (the LDS group table holds 1024;
    each of the 256 threads owns 4 entries): mostly empty groups, a few long ones,
    every element against the oracle."""
    rng = np.random.default_rng(E)
    sizes = np.zeros(E, dtype=np.int64)
    hot = rng.choice(E, 24, replace=False)
    sizes[hot] = rng.integers(1, 300, 24)
    sizes[E - 1] = 5                                   # the last group is not empty
    d = make_inputs(sizes=sizes, N=256, K=128, extra_rows=3, seed=E, device=DEV)
    print(f"E={E} rows={int(sizes.sum())}", flush=True)
    _check_full(d, f"E={E}")


@pytest.mark.parametrize("K", [320, 328])
def test_fwd_schedules_agree(K):
    """fwd loads stages in pairs when the rows average at least 2048 per expert
    and one by one otherwise (a launch choice from m_rows and the group count);
    padding rows past the last group switch it without changing any group, and
    both schedules sum in the same order, so the outputs agree bit for bit.  K =
    328 also runs the masked last stage under both."""
    sizes = [700, 300, 1100]
    d = make_inputs(sizes=sizes, N=512, K=K, extra_rows=3 * 2048 - 2100, seed=51, device=DEV)
    t = int(np.sum(sizes))
    assert d["M"] >= 2048 * 3                       # paired schedule
    y_pairs = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    y_single = mdg.grouped_det_gemm_fwd(d["x"][:t].contiguous(), d["w"], d["offs"])   # M = t < 2048 * 3
    torch.cuda.synchronize()
    assert torch.equal(y_pairs[:t].view(torch.int16), y_single.view(torch.int16))
    X, W = bits(d["x"][:t]), bits(d["w"])
    e = group_errs(values(y_single), oracle.fwd(X, W, d["offs"].cpu().numpy())[:t], np.array(sizes))
    assert max(e) <= TOL_BF16
