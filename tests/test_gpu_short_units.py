"""wgrad units of fewer than 4 real 32-row stages (a group of at most 96 rows)
run without the stage ring: only their real stages are loaded and multiplied.
The ring would also run zero stages, whose products leave every accumulator bit
as it is, so both must give the same dW bits.  A group padded with zero rows of
G and X to at least 97 rows has the same dW and runs through the ring: the two
launches are compared bit for bit in every output mode, and the short one
against the oracle.
"""
import numpy as np
import pytest
import torch

import moe_ragged_bf16_amd as mdg
import oracle
from workloads import make_inputs
from _parity import TOL_FP32, bits, block_err, ranges

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# 1, 2 and 3 real stages (1..32, 33..64, 65..96 rows), the 96/97 boundary, empty
# groups, and ring units (97, 128, 300 rows) in the same launch.
SIZES = [1, 17, 31, 32, 33, 0, 64, 65, 95, 96, 97, 128, 5, 300, 0]


def _padded(t, sizes, rows):
    """t's groups, each non-empty one followed by zero rows up to `rows` rows."""
    parts = []
    for (s, e), m in zip(ranges(sizes), sizes):
        parts.append(t[s:e])
        if 0 < m < rows:
            parts.append(torch.zeros((rows - m, t.shape[1]), dtype=t.dtype, device=t.device))
    return torch.cat(parts, 0)


@pytest.mark.parametrize("N,K", [(520, 264), (256, 256), (1032, 72)])
def test_short_units_match_the_ring_bitwise(N, K):
    d = make_inputs(sizes=SIZES, N=N, K=K, seed=21, device=DEV, tensors=("x", "g", "main_grad"))
    E = d["E"]
    psizes = [max(m, 97) if m > 0 else 0 for m in SIZES]
    assert all(m == 0 or m >= 97 for m in psizes)
    offs_p = torch.tensor(np.cumsum(psizes), dtype=torch.int32, device=DEV)
    g_p, x_p = _padded(d["g"], SIZES, 97), _padded(d["x"], SIZES, 97)
    assert g_p.shape[0] == sum(psizes)
    print(f"N={N} K={K} sizes={SIZES}", flush=True)

    mg32 = d["main_grad"]
    mg16 = mg32.to(torch.bfloat16)
    res = {}
    for tag, (g, x, offs) in (("short", (d["g"], d["x"], d["offs"])), ("ring", (g_p, x_p, offs_p))):
        dw32 = mdg.grouped_det_gemm_wgrad(g, x, offs, out_dtype=torch.float32)
        dw16 = mdg.grouped_det_gemm_wgrad(g, x, offs, out_dtype=torch.bfloat16)
        a32, a16 = mg32.clone(), mg16.clone()
        mdg.grouped_det_gemm_wgrad(g, x, offs, out=a32, accumulate=True)
        mdg.grouped_det_gemm_wgrad(g, x, offs, out=a16, accumulate=True)
        res[tag] = [dw32.view(torch.int32), dw16.view(torch.int16), a32.view(torch.int32), a16.view(torch.int16)]
    torch.cuda.synchronize()
    for name, a, b in zip(("fp32", "bf16", "fp32 accumulate", "bf16 accumulate"), res["short"], res["ring"]):
        assert torch.equal(a, b), name

    dw = res["short"][0].view(torch.float32).cpu().numpy()
    G, X = bits(d["g"]), bits(d["x"])
    for e, (s, t) in enumerate(ranges(SIZES)):
        if t == s:
            assert np.all(dw[e].view(np.int32) == 0), e
            continue
        ref = oracle.wgrad_expert(G[s:t], X[s:t])
        assert block_err(dw[e].astype(np.float64), ref) <= TOL_FP32, e
    assert dw.shape == (E, N, K)
