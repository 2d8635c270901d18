"""The allocation-free fwd entry point (grouped_det_gemm_fwd_noalloc), called
through the C ABI, against grouped_det_gemm_fwd with a caller workspace: two
calls in a row, the second with a smaller input, bit for bit and within the
oracle tolerance.  Both cases cut tail units, so the static scratch array
holds partial tiles and the plan; the second call must not see the first's."""
import numpy as np
import pytest
import torch

import moe_ragged_bf16_amd as mdg
import oracle
from moe_ragged_bf16_amd import _capi
from workloads import make_inputs
from _parity import TOL_BF16, bits, group_errs, values
from _plan import tail_plan

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENTINEL = 0x7FC1

CASES = [
    ([300, 700, 0, 1900], 1088, 1000, 3),   # partial n tile, partial last stage, padding rows
    ([100, 50], 256, 512, 2),               # smaller
]


def _noalloc(x, w, offs, y):
    M, K = x.shape
    E, N, _ = w.shape
    st = _capi.load_library().grouped_det_gemm_fwd_noalloc(
        x.data_ptr(), w.data_ptr(), offs.data_ptr(), y.data_ptr(), M, N, K, E,
        torch.cuda.current_stream().cuda_stream)
    _capi.check("grouped_det_gemm_fwd_noalloc", st)


def test_noalloc_fwd_equals_fwd_on_consecutive_calls():
    for i, (sizes, N, K, pad) in enumerate(CASES):
        d = make_inputs(sizes=sizes, N=N, K=K, extra_rows=pad, seed=70 + i, device=DEV)
        M, E = d["M"], d["E"]
        print(f"noalloc fwd: sizes={sizes} N={N} K={K} M={M}", flush=True)
        assert tail_plan("fwd", sizes, N, K, M, E)[2] >= 2          # the tail split (and the scratch) is used
        ws = torch.empty(mdg.fwd_workspace_bytes(M, N, K, E), dtype=torch.uint8, device=DEV)
        ref = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"], workspace=ws)
        y = torch.full((M, N), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        torch.cuda.synchronize()
        reserved = torch.cuda.memory_reserved()
        _noalloc(d["x"], d["w"], d["offs"], y)
        torch.cuda.synchronize()
        assert torch.cuda.memory_reserved() == reserved
        t = int(np.sum(sizes))
        assert torch.equal(y[:t].view(torch.int16), ref[:t].view(torch.int16))
        assert torch.all(y[t:].view(torch.int16) == SENTINEL)      # padding rows untouched
        e = group_errs(values(y[:t]), oracle.fwd(bits(d["x"]), bits(d["w"]), d["offs"].cpu().numpy())[:t],
                       np.asarray(sizes))
        assert max(e) <= TOL_BF16, e


def test_noalloc_fwd_refusals_and_empty():
    lib = _capi.load_library()
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((2, 256, 64), dtype=torch.bfloat16, device=DEV)
    offs = torch.tensor([4, 8], dtype=torch.int32, device=DEV)
    y = torch.zeros((8, 256), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    call = lambda **kw: lib.grouped_det_gemm_fwd_noalloc(
        kw.get("x", x.data_ptr()), w.data_ptr(), offs.data_ptr(), kw.get("y", y.data_ptr()),
        kw.get("M", 8), kw.get("N", 256), 64, 2, s)
    assert call(N=100) == _capi.MDG_EUNSUPPORTED
    assert call(y=x.data_ptr()) == _capi.MDG_EOVERLAP
    assert call(M=0, x=0, y=0) == _capi.MDG_OK
    torch.cuda.synchronize()
