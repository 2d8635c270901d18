"""The autograd wrapper on the GPU kernels: its outputs and gradients are the
one-shot entry points' bits, the fused accumulation gives AccumulateGrad's bits
of the deterministic dW (flashinfer PR #8924, "Fused weight-gradient
accumulation into main_grad"; its GPU test oracle is ``out0.add_(dW)`` in out's
dtype), and the padding rows get zeros.
"""
import numpy as np
import pytest
import torch

import moe_ragged_bf16_amd as mdg
import oracle
from workloads import make_inputs
from _parity import TOL_BF16, bits, block_err, group_errs, values

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SIZES = [0, 700, 1, 300, 0, 257]
PAD = 5


def _case(seed=11, N=512, K=320):
    d = make_inputs(sizes=SIZES, N=N, K=K, extra_rows=PAD, seed=seed, device=DEV,
                    tensors=("x", "w", "g", "main_grad"))
    d["t"] = int(np.sum(SIZES))
    return d


def _eq(a, b):
    v = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.contiguous().view(v), b.contiguous().view(v))


def test_unfused_matches_entry_points_and_oracle():
    d = _case()
    t, M = d["t"], d["M"]
    print(f"autograd unfused: sizes={SIZES} pad={PAD} N={d['N']} K={d['K']}", flush=True)
    x = d["x"].clone().requires_grad_()
    w = d["w"].clone().requires_grad_()
    y = mdg.cake_grouped_det_mm(x, w, d["offs"])
    y.backward(d["g"])
    torch.cuda.synchronize()
    y_ref = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    dx_ref = mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"])
    dw_ref = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.bfloat16)
    assert _eq(y.detach()[:t], y_ref[:t])
    assert _eq(x.grad[:t], dx_ref[:t])
    assert _eq(w.grad, dw_ref)
    assert torch.all(y.detach()[t:].view(torch.int16) == 0)          # +0.0 in the padding rows
    assert torch.all(x.grad[t:].view(torch.int16) == 0)
    # and against the oracle (fp64), per group
    offs = d["offs"].cpu().numpy()
    ry = oracle.fwd(bits(d["x"]), bits(d["w"]), offs)
    rdx = oracle.dgrad(bits(d["g"]), bits(d["w"]), offs)
    rdw = oracle.wgrad(bits(d["g"]), bits(d["x"]), offs)
    assert max(group_errs(values(y[:t]), ry[:t], SIZES)) < TOL_BF16
    assert max(group_errs(values(x.grad[:t]), rdx[:t], SIZES)) < TOL_BF16
    gw = values(w.grad)
    assert max(block_err(gw[e], rdw[e]) for e in range(len(SIZES))) < TOL_BF16


def test_m_indptr_and_offs_forms_agree():
    d = _case(seed=12)
    a = mdg.cake_grouped_det_mm(d["x"], d["w"], d["offs"])
    b = mdg.cake_grouped_det_mm(d["x"], d["w"], d["m_indptr"])
    assert _eq(a, b)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fused_equals_accumulate_grad_of_det_dw(dtype):
    """main_grad after the fused backward == main_grad0.add_(dW) in its dtype,
    and == autograd's own AccumulateGrad of the unfused backward's dW."""
    d = _case(seed=13)
    print(f"autograd fused: main_grad {dtype}", flush=True)
    R = mdg.wgrad_chunk_rows(d["M"], d["N"], d["K"], len(SIZES))
    assert max(SIZES) > R and any(0 < s <= R for s in SIZES)   # split and unsplit experts
    mg0 = d["main_grad"].to(dtype)
    mg0[0, :2, :3] = -0.0                                         # empty expert: -0.0 + 0.0 = +0.0
    x = d["x"].clone().requires_grad_()
    w = d["w"].clone().requires_grad_()
    w.main_grad = mg0.clone()
    mdg.cake_grouped_det_mm(x, w, d["offs"], fuse_wgrad_accumulation=True).backward(d["g"])
    dw = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=dtype)
    assert _eq(w.main_grad, mg0.clone().add_(dw))
    assert w.grad is None
    # autograd's AccumulateGrad: an unfused backward into a w.grad holding main_grad0
    # (fp32 main_grad: w's dtype is bf16, so the comparison is the fp32 add above)
    if dtype == torch.bfloat16:
        w2 = d["w"].clone().requires_grad_()
        w2.grad = mg0.clone()
        mdg.cake_grouped_det_mm(d["x"], w2, d["offs"]).backward(d["g"])
        assert _eq(w.main_grad, w2.grad)
        want = oracle.accumulate_bf16(bits(mg0), bits(dw))
        assert np.array_equal(bits(w.main_grad), want)
    else:
        want = oracle.accumulate_fp32(mg0.cpu().numpy(), dw.cpu().numpy())
        assert np.array_equal(w.main_grad.cpu().numpy().view(np.uint32), want.view(np.uint32))
    assert not torch.signbit(w.main_grad[0, :2, :3].float()).any()


def test_placeholder_retain_graph_and_reruns():
    d = _case(seed=14)
    x = d["x"].clone().requires_grad_()
    w = d["w"].clone().requires_grad_()
    w.main_grad = d["main_grad"].clone()
    w.grad_added_to_main_grad = False
    w.zero_out_wgrad = True
    y = mdg.cake_grouped_det_mm(x, w, d["offs"], fuse_wgrad_accumulation=True)
    y.backward(d["g"], retain_graph=True)
    assert w.grad_added_to_main_grad is True
    assert w.grad.shape == w.shape and w.grad.dtype == torch.bfloat16 and torch.all(w.grad == 0)
    y.backward(d["g"])                                            # adds a second time
    dw = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)
    assert _eq(w.main_grad, d["main_grad"].clone().add_(dw).add_(dw))
    # run to run: a fresh graph gives the same bits
    for _ in range(3):
        w.main_grad = d["main_grad"].clone()
        x.grad = None
        mdg.cake_grouped_det_mm(x, w, d["offs"], fuse_wgrad_accumulation=True).backward(d["g"])
        assert _eq(w.main_grad, d["main_grad"].clone().add_(dw))


def test_strided_main_grad_and_deterministic_mode():
    d = _case(seed=15, N=256, K=128)
    E, N, K = d["w"].shape
    big = torch.randn(E, 2 * N, K, device=DEV)
    before = big.clone()
    w = d["w"].clone().requires_grad_()
    w.main_grad = big[:, N:]
    prev = torch.are_deterministic_algorithms_enabled()
    torch.use_deterministic_algorithms(True)
    try:
        mdg.cake_grouped_det_mm(d["x"], w, d["offs"], fuse_wgrad_accumulation=True).backward(d["g"])
    finally:
        torch.use_deterministic_algorithms(prev)
    dw = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)
    assert _eq(big[:, :N], before[:, :N])
    assert _eq(big[:, N:], before[:, N:] + dw)
