"""The fwd/dgrad tail split on the GPU: parity with the oracle for cases with 8,
3, 4 or 7 pieces per tail unit and without a split (also with a reduction that
ends in a partial stage), the plan the kernel writes against the documented
rule, bitwise reruns, a workspace reused across calls of different sizes, and
what regrouping and permuting experts leave bitwise unchanged.

Reading stated here: a unit's output bits are a function of its operands and
of its piece count (1 when whole); the split is decided from the total unit
count U (the last U mod 256 units are cut), so a row's bits can change when
other groups change, exactly where its unit's piece count changes."""
import numpy as np
import pytest
import torch

import moe_ragged_bf16_amd as mdg
import oracle
from workloads import make_inputs
from _parity import TOL_BF16, bits, group_errs, values
from _plan import split_mask, tail_plan

DEV = "cuda:0"

# (group sizes, N, K, padding rows, expected pieces per tail unit by op)
CASES = [
    ([300, 700], 512, 1024, 3, {"fwd": 8, "dgrad": 4}),
    ([2304], 2048, 512, 0, {"fwd": 3}),
    ([4352], 2048, 256, 0, {"fwd": 1, "dgrad": 8}),
    ([0, 511, 1, 0, 257], 768, 384, 9, {}),
    ([4352], 1088, 320, 2, {"fwd": 3, "dgrad": 7}),      # partial n tiles, split tail
    # k (fwd) and n (dgrad) not multiples of 32: the last piece ends in a partial stage
    ([300, 700], 512, 1000, 3, {"fwd": 8, "dgrad": 4}),
    ([4352], 1032, 328, 2, {"fwd": 3, "dgrad": 7}),
]


def _run(d, ws_f=None, ws_d=None):
    y = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"], workspace=ws_f)
    dx = mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"], workspace=ws_d)
    torch.cuda.synchronize()
    return y, dx


def _workspaces(M, N, K, E):
    return (torch.empty(mdg.fwd_workspace_bytes(M, N, K, E), dtype=torch.uint8, device=DEV),
            torch.empty(mdg.dgrad_workspace_bytes(M, N, K, E), dtype=torch.uint8, device=DEV))


def _written_plan(ws):
    """(T, S) as the GEMM kernel wrote it at the head of its workspace."""
    h = ws[:8].view(torch.int32).cpu()
    return int(h[0]), int(h[1])


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-N{c[1]}-K{c[2]}" for c in CASES])
def test_tail_split_parity(case):
    sizes, N, K, pad, pieces = case
    d = make_inputs(sizes=sizes, N=N, K=K, extra_rows=pad, seed=11, device=DEV)
    ws_f, ws_d = _workspaces(d["M"], N, K, d["E"])
    y, dx = _run(d, ws_f, ws_d)
    # the plan the kernels used is the documented rule's, and the case splits as intended
    for op, ws in (("fwd", ws_f), ("dgrad", ws_d)):
        _, T, S = tail_plan(op, sizes, N, K, d["M"], d["E"])
        assert _written_plan(ws) == (T, S), (op, _written_plan(ws), (T, S))
        if op in pieces:
            assert S == pieces[op], (op, S)
    X, W, G = bits(d["x"]), bits(d["w"]), bits(d["g"])
    offs = d["offs"].cpu().numpy()
    Mg = int(np.sum(sizes))
    ey = group_errs(values(y[:Mg]), oracle.fwd(X, W, offs)[:Mg], np.array(sizes))
    edx = group_errs(values(dx[:Mg]), oracle.dgrad(G, W, offs)[:Mg], np.array(sizes))
    assert max(ey, default=0) <= TOL_BF16, ("fwd", ey)
    assert max(edx, default=0) <= TOL_BF16, ("dgrad", edx)


@pytest.mark.gpu
def test_tail_split_reruns_bitwise_with_poisoned_workspace():
    sizes, N, K, pad, _ = CASES[0]
    d = make_inputs(sizes=sizes, N=N, K=K, extra_rows=pad, seed=12, device=DEV)
    M, E = d["M"], d["E"]
    ws_f = torch.empty(mdg.fwd_workspace_bytes(M, N, K, E), dtype=torch.uint8, device=DEV)
    ws_d = torch.empty(mdg.dgrad_workspace_bytes(M, N, K, E), dtype=torch.uint8, device=DEV)
    first = None
    for it in range(5):
        ws_f.random_(0, 256)
        ws_d.random_(0, 256)
        y, dx = _run(d, ws_f, ws_d)
        Mg = int(np.sum(sizes))        # padding rows of a fresh output are left uninitialised
        cur = (y[:Mg].view(torch.int16).clone(), dx[:Mg].view(torch.int16).clone())
        if first is None:
            first = cur
        else:
            assert torch.equal(first[0], cur[0]) and torch.equal(first[1], cur[1]), it


@pytest.mark.gpu
def test_workspace_reused_across_sizes():
    a = make_inputs(sizes=CASES[0][0], N=CASES[0][1], K=CASES[0][2], seed=13, device=DEV)
    b = make_inputs(sizes=CASES[2][0], N=CASES[2][1], K=CASES[2][2], seed=14, device=DEV)
    need = max(mdg.fwd_workspace_bytes(t["M"], t["N"], t["K"], t["E"]) for t in (a, b))
    need = max(need, max(mdg.dgrad_workspace_bytes(t["M"], t["N"], t["K"], t["E"]) for t in (a, b)))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    ra, rb = _run(a), _run(b)                       # fresh workspaces
    sa = _run(a, ws, ws)                            # one shared workspace, calls in stream order
    sb = _run(b, ws, ws)
    for r, s in ((ra, sa), (rb, sb)):
        assert torch.equal(r[0].view(torch.int16), s[0].view(torch.int16))
        assert torch.equal(r[1].view(torch.int16), s[1].view(torch.int16))


def _outputs(sizes, x, w, g, N, K):
    """fwd and dgrad of one arrangement, with the plans the kernels wrote."""
    E, M = len(sizes), x.shape[0]
    offs = torch.tensor(np.cumsum(sizes), dtype=torch.int32, device=DEV)
    ws_f, ws_d = _workspaces(M, N, K, E)
    y = mdg.grouped_det_gemm_fwd(x, w, offs, workspace=ws_f)
    dx = mdg.grouped_det_gemm_dgrad(g, w, offs, workspace=ws_d)
    torch.cuda.synchronize()
    return {"fwd": (y, _written_plan(ws_f)), "dgrad": (dx, _written_plan(ws_d))}


def _compare(op, a, b, sizes_a, sizes_b, rows_b, N, K, ref):
    """a (arrangement A) against b (arrangement B, its rows reordered by rows_b
    into A's order): bitwise wherever the element's unit has the same piece count
    in both, within tolerance of the oracle everywhere.  Returns the number of
    elements compared bitwise and the number whose piece count differs."""
    M = int(np.sum(sizes_a))
    out_a, plan_a = a
    out_b, plan_b = b
    ma, pa = split_mask(op, sizes_a, N, K)
    mb, pb = split_mask(op, sizes_b, N, K)
    assert plan_a == pa[1:] and plan_b == pb[1:], (op, plan_a, pa, plan_b, pb)
    pieces_a = np.where(ma, pa[2], 1)
    pieces_b = np.where(mb, pb[2], 1)[rows_b]
    same = np.repeat(pieces_a == pieces_b, 256, axis=1)[:, :out_a.shape[1]]
    ga = bits(out_a[:M])
    gb = bits(out_b[:M][torch.from_numpy(rows_b).to(DEV)])
    assert np.array_equal(ga[same], gb[same]), op
    for g_ in (ga, gb):
        e = group_errs(oracle.widen_bf16(g_).astype(np.float64), ref, np.asarray(sizes_a))
        assert max(e) <= TOL_BF16, (op, e)
    return int(same.sum()), int((~same).sum())


@pytest.mark.gpu
def test_regrouping_and_permutation_bits():
    """Splitting a group into two consecutive groups that share its weight, and
    permuting the experts (weights, groups and their rows), change no output bit
    of a unit whose piece count stays the same.  The first arrangement has
    exactly 256 fwd units (no split); regrouping makes 264, so the last 8 fwd
    units are cut in 8 and only their rows may differ in the last bits."""
    N, K = 2048, 1024
    base = [2000, 3000, 3000]
    regroup = [2000, 1100, 1900, 3000]          # group 1 of base, split in two
    perm = [2, 0, 1]
    d = make_inputs(sizes=base, N=N, K=K, seed=61, device=DEV)
    x, w, g = d["x"], d["w"], d["g"]
    starts = np.concatenate([[0], np.cumsum(base)])
    refs = {"fwd": oracle.fwd(bits(x), bits(w), d["offs"].cpu().numpy()),
            "dgrad": oracle.dgrad(bits(g), bits(w), d["offs"].cpu().numpy())}
    A = _outputs(base, x, w, g, N, K)
    # regrouping: same rows, weights [W0, W1, W1, W2]
    R = _outputs(regroup, x, w[[0, 1, 1, 2]].contiguous(), g, N, K)
    # permutation: groups (and their rows) in the order perm, weights W[perm]
    rows_p = np.concatenate([np.arange(starts[e], starts[e + 1]) for e in perm])
    inv = np.argsort(rows_p)                      # arrangement P row -> base row order
    rp = torch.from_numpy(rows_p).to(DEV)
    P = _outputs([base[e] for e in perm], x[rp].contiguous(), w[perm].contiguous(), g[rp].contiguous(), N, K)
    ident = np.arange(int(np.sum(base)))
    counts = {}
    for op in ("fwd", "dgrad"):
        counts[(op, "regroup")] = _compare(op, A[op], R[op], base, regroup, ident, N, K, refs[op])
        counts[(op, "perm")] = _compare(op, A[op], P[op], base, [base[e] for e in perm], inv, N, K, refs[op])
    print(counts, flush=True)
    # both sides of the rule occur: fwd regrouping changes the piece count of some units
    assert counts[("fwd", "regroup")][1] > 0 and counts[("fwd", "regroup")][0] > 0
    assert counts[("fwd", "perm")][1] == 0 and counts[("dgrad", "perm")][1] == 0
