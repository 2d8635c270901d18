"""The fwd/dgrad tail split on the GPU: parity with the oracle for cases with 8,
3, 4 or 7 pieces per tail unit and without a split (also with a reduction that
ends in a partial stage), bitwise reruns, and a workspace
reused across calls of different sizes."""
import numpy as np
import pytest
import torch

import moe_ragged_bf16_amd as mdg
import oracle
from workloads import make_inputs
from _parity import TOL_BF16, bits, group_errs, values

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


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-N{c[1]}-K{c[2]}" for c in CASES])
def test_tail_split_parity(case):
    sizes, N, K, pad, _ = case
    d = make_inputs(sizes=sizes, N=N, K=K, extra_rows=pad, seed=11, device=DEV)
    y, dx = _run(d)
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
