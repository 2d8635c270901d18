"""Prepared launches on the GPU (Cake ragged BF16 grouped GEMM API page,
"Prepared launches"; flashinfer PR #8924, "API" and "Tests"): the same bits as
the one-shot functions, offsets rewritten in place, HIP graph capture and
replays (each replay checked against eager results, with eager work and
synchronisations between replays), the version counter and no allocation.
"""
import numpy as np
import pytest
import torch

import moe_ragged_bf16_amd as mdg
from workloads import make_inputs, offsets_from_sizes

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SIZES = [300, 0, 700, 1, 257]
SIZES2 = [0, 900, 100, 250, 8]      # same total rows, other routing


def _case(seed=21, N=512, K=320, pad=3):
    d = make_inputs(sizes=SIZES, N=N, K=K, extra_rows=pad, seed=seed, device=DEV,
                    tensors=("x", "w", "g", "main_grad"))
    d["t"] = int(np.sum(SIZES))
    return d


def _eq(a, b):
    v = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.contiguous().view(v), b.contiguous().view(v))


def test_prepared_equals_one_shot_and_reruns():
    d = _case()
    t = d["t"]
    print(f"prepared launches: sizes={SIZES}", flush=True)
    lf = mdg.prepare_grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    ld = mdg.prepare_grouped_det_gemm_dgrad(d["g"], d["w"], d["m_indptr"])
    lw32 = mdg.prepare_grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)
    lw16 = mdg.prepare_grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"])
    assert lf.plan["op"] == "fwd" and lf.plan["kernels"] in (1, 2) and lf.plan["accumulate"] == "off"
    assert lw32.plan["kernels"] == 2 and lw32.plan["chunk_rows"] >= 256    # GEMM + chunk reduce
    y1 = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    dx1 = mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"])
    dw32 = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)
    dw16 = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"])
    for _ in range(3):
        for l in (lf, ld, lw32, lw16):
            l.out.view(torch.uint8).fill_(0xFF)        # poison: every launch rewrites
            l.launch()
        torch.cuda.synchronize()
        assert _eq(lf.out[:t], y1[:t]) and _eq(ld.out[:t], dx1[:t])
        assert _eq(lw32.out, dw32) and _eq(lw16.out, dw16)


def test_offsets_rewritten_in_place_between_launches():
    d = _case(seed=22)
    lf = mdg.prepare_grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    lw = mdg.prepare_grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)
    lf.launch()
    lw.launch()
    d["offs"].copy_(torch.from_numpy(offsets_from_sizes(SIZES2)).to(DEV))
    y2 = lf.launch()
    dw2 = lw.launch()
    offs2 = torch.from_numpy(offsets_from_sizes(SIZES2)).to(DEV)
    y_ref = mdg.grouped_det_gemm_fwd(d["x"], d["w"], offs2)
    dw_ref = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], offs2, out_dtype=torch.float32)
    torch.cuda.synchronize()
    t = int(np.sum(SIZES2))
    assert _eq(y2[:t], y_ref[:t]) and _eq(dw2, dw_ref)
    assert torch.all(dw2[0] == 0)                        # expert 0 is empty now


@pytest.mark.parametrize("mg_dtype", [torch.float32, torch.bfloat16])
def test_graph_capture_and_replays(mg_dtype):
    d = _case(seed=23)
    t = d["t"]
    print(f"graph capture: main_grad {mg_dtype}", flush=True)
    mg0 = d["main_grad"].to(mg_dtype)
    mg = mg0.clone()
    lf = mdg.prepare_grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    ld = mdg.prepare_grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"])
    lw = mdg.prepare_grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out=mg, accumulate=True)
    assert lw.plan["accumulate"] == "fused"
    y_ref = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    dx_ref = mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"])
    dw = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=mg_dtype)
    torch.cuda.synchronize()
    v0 = mg._version
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lf.launch()
        ld.launch()
        lw.launch()
    torch.cuda.synchronize()
    assert _eq(mg, mg0)                                 # capture runs nothing
    assert mg._version == v0 + 1                        # ... but bumps the version once
    expect = mg0.clone()
    for r in range(3):
        lf.out.zero_()                                  # eager work between replays
        ld.out.view(torch.uint8).fill_(0x7F)
        graph.replay()
        expect.add_(dw)                                 # AccumulateGrad bits, once per replay
        torch.cuda.synchronize()
        assert _eq(lf.out[:t], y_ref[:t]), r
        assert _eq(ld.out[:t], dx_ref[:t]), r
        assert _eq(mg, expect), r
        assert mg._version == v0 + 1                    # replays run no Python
        mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])   # unrelated eager launch
        torch.cuda.synchronize()
    # offsets rewritten in place between replays
    offs2 = torch.from_numpy(offsets_from_sizes(SIZES2)).to(DEV)
    d["offs"].copy_(offs2)
    graph.replay()
    y2 = mdg.grouped_det_gemm_fwd(d["x"], d["w"], offs2)
    torch.cuda.synchronize()
    t2 = int(np.sum(SIZES2))
    assert _eq(lf.out[:t2], y2[:t2])


def test_launch_allocates_nothing_and_bumps_version():
    d = _case(seed=24)
    mg = d["main_grad"].clone()
    ls = [mdg.prepare_grouped_det_gemm_fwd(d["x"], d["w"], d["offs"]),
          mdg.prepare_grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"]),
          mdg.prepare_grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out=mg, accumulate=True)]
    for l in ls:
        l.launch()
    torch.cuda.synchronize()
    a0 = torch.cuda.memory_allocated()
    free0 = torch.cuda.mem_get_info()[0]
    v0 = mg._version
    for _ in range(5):
        for l in ls:
            l.launch()
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == a0
    assert torch.cuda.mem_get_info()[0] == free0
    assert mg._version == v0 + 5


def test_zero_rows_launches():
    E, N, K = 3, 256, 64
    x = torch.empty((0, K), dtype=torch.bfloat16, device=DEV)
    g = torch.empty((0, N), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((E, N, K), dtype=torch.bfloat16, device=DEV)
    offs = torch.zeros(E, dtype=torch.int32, device=DEV)
    lf = mdg.prepare_grouped_det_gemm_fwd(x, w, offs)
    assert lf.plan["kernels"] == 0 and lf.launch().shape == (0, N)
    mg = torch.randn((E, N, K), device=DEV)
    before = mg.clone()
    la = mdg.prepare_grouped_det_gemm_wgrad(g, x, offs, out=mg, accumulate=True)
    assert la.plan["kernels"] == 0
    la.launch()
    lo = mdg.prepare_grouped_det_gemm_wgrad(g, x, offs, out_dtype=torch.float32)
    assert lo.plan["kernels"] == 1                      # overwrite: zeros
    lo.out.fill_(1.0)
    lo.launch()
    torch.cuda.synchronize()
    assert _eq(mg, before) and torch.all(lo.out.view(torch.int32) == 0)
