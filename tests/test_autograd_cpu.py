"""The autograd wrapper's host logic on the CPU: the Megatron main_grad
convention, its checks and refusals (flashinfer PR #8924, "Fused
weight-gradient accumulation into main_grad"), with the device entry points
replaced by oracle-backed stand-ins (tests/_standins.py).  The same contract
runs on the GPU kernels in test_gpu_autograd.py.
"""
import numpy as np
import pytest
import torch
from torch.utils.checkpoint import checkpoint

import oracle
from moe_ragged_bf16_amd import CakeGroupedDetMm, cake_grouped_det_mm
from workloads import make_inputs
from _standins import install, _bits, _bf16, _offs

SIZES = [3, 0, 5, 4]


@pytest.fixture
def case(monkeypatch):
    s = install(monkeypatch)
    d = make_inputs(sizes=SIZES, K=16, N=8, extra_rows=2, seed=3, tensors=("x", "w", "g", "main_grad"))
    x = d["x"].clone().requires_grad_()
    w = d["w"].clone().requires_grad_()
    d.update(x=x, w=w, dy=d["g"], s=s)
    return d


def _refs(d):
    x, w, dy, offs = d["x"], d["w"], d["dy"], d["offs"].numpy()
    t = int(offs[-1])
    y = oracle.fwd(_bits(x), _bits(w), offs, precision="fp32")
    dx = oracle.dgrad(_bits(dy), _bits(w), offs, precision="fp32")
    y[t:] = 0
    dx[t:] = 0
    dw32 = oracle.wgrad(_bits(dy), _bits(x), offs, precision="fp32").astype(np.float32)
    return _bf16(y), _bf16(dx), dw32


def _eq(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_unfused_gradients(case):
    y_ref, dx_ref, dw32 = _refs(case)
    y = cake_grouped_det_mm(case["x"], case["w"], case["offs"])
    assert _eq(y.detach(), y_ref)
    assert torch.all(y.detach()[12:] == 0)                  # rows past the last group
    y.backward(case["dy"])
    assert _eq(case["x"].grad, dx_ref)
    assert _eq(case["w"].grad, _bf16(dw32))                 # w's dtype: the overwrite dW rounded once
    assert case["s"].calls == ["fwd", "zero_pad_rows", "dgrad", "zero_pad_rows", "wgrad"]


def test_m_indptr_form(case):
    y = cake_grouped_det_mm(case["x"], case["w"], case["m_indptr"])
    y_ref, _, _ = _refs(case)
    assert _eq(y.detach(), y_ref)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fused_adds_into_main_grad_and_returns_none(case, dtype):
    _, dx_ref, dw32 = _refs(case)
    w = case["w"]
    w.main_grad = case["main_grad"].to(dtype)
    mg0 = w.main_grad.clone()
    v0 = w.main_grad._version
    y = cake_grouped_det_mm(case["x"], w, case["offs"], fuse_wgrad_accumulation=True)
    y.backward(case["dy"])
    if dtype == torch.float32:
        want = torch.from_numpy(oracle.accumulate_fp32(mg0.numpy(), dw32))
    else:
        want = torch.from_numpy(oracle.accumulate_bf16(_bits(mg0), oracle.round_bf16_rne(dw32)).view(np.int16)) \
            .view(torch.bfloat16)
    assert _eq(w.main_grad, want)
    assert w.grad is None                                   # no grad_added_to_main_grad attribute
    assert _eq(case["x"].grad, dx_ref)
    assert w.main_grad._version > v0
    assert "wgrad_acc" in case["s"].calls and "wgrad" not in case["s"].calls


@pytest.mark.parametrize("zero_out", [False, True, None])
def test_placeholder_with_grad_added_to_main_grad(case, zero_out):
    w = case["w"]
    w.main_grad = case["main_grad"]
    w.grad_added_to_main_grad = False
    if zero_out is not None:
        w.zero_out_wgrad = zero_out
    cake_grouped_det_mm(case["x"], w, case["offs"], fuse_wgrad_accumulation=True).backward(case["dy"])
    assert w.grad_added_to_main_grad is True
    assert w.grad is not None and w.grad.shape == w.shape and w.grad.dtype == w.dtype
    if zero_out:
        assert torch.all(w.grad == 0)


def test_retain_graph_adds_twice(case):
    _, _, dw32 = _refs(case)
    w = case["w"]
    w.main_grad = case["main_grad"]
    mg0 = w.main_grad.clone().numpy()
    y = cake_grouped_det_mm(case["x"], w, case["offs"], fuse_wgrad_accumulation=True)
    y.backward(case["dy"], retain_graph=True)
    y.backward(case["dy"])
    want = oracle.accumulate_fp32(oracle.accumulate_fp32(mg0, dw32), dw32)
    assert _eq(w.main_grad, torch.from_numpy(want))


def test_autograd_grad_without_w_still_adds(case):
    _, dx_ref, dw32 = _refs(case)
    w = case["w"]
    w.main_grad = case["main_grad"]
    mg0 = w.main_grad.clone().numpy()
    y = cake_grouped_det_mm(case["x"], w, case["offs"], fuse_wgrad_accumulation=True)
    (gx,) = torch.autograd.grad(y, [case["x"]], case["dy"])
    assert _eq(gx, dx_ref)
    assert _eq(w.main_grad, torch.from_numpy(oracle.accumulate_fp32(mg0, dw32)))


def test_frozen_w_gets_nothing(case):
    w = case["w"].detach()
    w.main_grad = case["main_grad"]
    mg0 = w.main_grad.clone()
    y = cake_grouped_det_mm(case["x"], w, case["offs"], fuse_wgrad_accumulation=True)
    y.backward(case["dy"])
    assert _eq(w.main_grad, mg0)
    assert case["x"].grad is not None
    assert not any(c.startswith("wgrad") for c in case["s"].calls)


def test_repointed_main_grad_receives_the_add(case):
    _, _, dw32 = _refs(case)
    w = case["w"]
    first = case["main_grad"].clone()
    w.main_grad = first
    y = cake_grouped_det_mm(case["x"], w, case["offs"], fuse_wgrad_accumulation=True)
    second = torch.full_like(first, 0.5)
    w.main_grad = second
    y.backward(case["dy"])
    assert _eq(first, case["main_grad"])
    assert _eq(second, torch.from_numpy(oracle.accumulate_fp32(np.full(first.shape, 0.5, np.float32), dw32)))


@pytest.mark.parametrize("fuse", [False, True])
def test_create_graph_refused(case, fuse):
    w = case["w"]
    w.main_grad = case["main_grad"]
    y = cake_grouped_det_mm(case["x"], w, case["offs"], fuse_wgrad_accumulation=fuse)
    with pytest.raises(NotImplementedError):
        torch.autograd.grad(y, [case["x"], w], case["dy"], create_graph=True)


@pytest.mark.filterwarnings("ignore:`torch.jit.trace` is deprecated:DeprecationWarning")
def test_trace_refused(case):
    with pytest.raises(NotImplementedError):
        torch.jit.trace(lambda a, b: cake_grouped_det_mm(a, b, case["offs"]), (case["x"], case["w"]))


def test_compile_refused_or_run_eagerly(case):
    y_ref, _, _ = _refs(case)
    f = lambda a, b: cake_grouped_det_mm(a, b, case["offs"])  # noqa: E731
    with pytest.raises(Exception, match="NotImplementedError|cannot be compiled|Observed exception"):
        torch.compile(f, backend="eager", fullgraph=True)(case["x"], case["w"])
    torch._dynamo.reset()
    y = torch.compile(f, backend="eager")(case["x"], case["w"])   # falls back to running eagerly
    assert _eq(y.detach(), y_ref)


def test_reentrant_checkpoint_refused(case):
    w = case["w"]
    w.main_grad = case["main_grad"]
    y = checkpoint(lambda a, b: cake_grouped_det_mm(a, b, case["offs"], fuse_wgrad_accumulation=True),
                   case["x"], w, use_reentrant=True)
    with pytest.raises(ValueError, match="main_grad"):
        y.backward(case["dy"])


def test_non_reentrant_checkpoint_adds_once(case):
    _, dx_ref, dw32 = _refs(case)
    w = case["w"]
    w.main_grad = case["main_grad"]
    mg0 = w.main_grad.clone().numpy()
    w.grad_added_to_main_grad = False
    y = checkpoint(lambda a, b: cake_grouped_det_mm(a, b, case["offs"], fuse_wgrad_accumulation=True),
                   case["x"], w, use_reentrant=False)
    y.backward(case["dy"])
    assert _eq(w.main_grad, torch.from_numpy(oracle.accumulate_fp32(mg0, dw32)))
    assert _eq(case["x"].grad, dx_ref)
    assert w.grad_added_to_main_grad is True
    assert case["s"].calls.count("fwd") == 2 and case["s"].calls.count("wgrad_acc") == 1


def test_nested_non_reentrant_checkpoints(case):
    _, _, dw32 = _refs(case)
    w = case["w"]
    w.main_grad = case["main_grad"]
    mg0 = w.main_grad.clone().numpy()
    inner = lambda a, b: cake_grouped_det_mm(a, b, case["offs"], fuse_wgrad_accumulation=True)  # noqa: E731
    outer = lambda a, b: checkpoint(inner, a, b, use_reentrant=False)  # noqa: E731
    checkpoint(outer, case["x"], w, use_reentrant=False).backward(case["dy"])
    assert _eq(w.main_grad, torch.from_numpy(oracle.accumulate_fp32(mg0, dw32)))


def test_apply_argument_rules(case):
    x, w, offs = case["x"], case["w"], case["offs"]
    for stale in (True, False, 0):
        with pytest.raises(TypeError):
            CakeGroupedDetMm.apply(x, w, offs, stale)
    for bad in (1, None, "True", 0.0):
        with pytest.raises(ValueError):
            CakeGroupedDetMm.apply(x, w, offs, None, bad)
    with pytest.raises(TypeError):
        cake_grouped_det_mm(x, w, offs, deterministic=True)      # no mode argument
    with pytest.raises(TypeError):
        cake_grouped_det_mm(x, w, offs, True)                    # the flag is keyword-only
    y = CakeGroupedDetMm.apply(x, w, offs)                       # defaults: reserved slot None, no fusion
    y.backward(case["dy"])
    assert w.grad is not None


def test_main_grad_checks_at_recorded_forward(case):
    x, w, offs = case["x"], case["w"], case["offs"]
    E, N, K = w.shape
    with pytest.raises(ValueError, match="no main_grad"):
        cake_grouped_det_mm(x, w, offs, fuse_wgrad_accumulation=True)
    with torch.no_grad():                                         # not recorded: not checked
        cake_grouped_det_mm(x, w, offs, fuse_wgrad_accumulation=True)
    bad = {
        TypeError: [torch.zeros(E, N, K, dtype=torch.float16)],
        ValueError: [torch.zeros(E, N, K + 1)[..., :K].transpose(1, 2).contiguous().transpose(1, 2),  # K stride
                     torch.zeros(1, N, K).expand(E, N, K),                                           # experts alias
                     torch.zeros(E, 1, K).expand(E, N, K),                                           # rows alias
                     torch.zeros(E, N, K - 1),
                     torch.zeros(E + 1, N, K)],
    }
    for exc, mgs in bad.items():
        for mg in mgs:
            w.main_grad = mg
            with pytest.raises(exc):
                cake_grouped_det_mm(x, w, offs, fuse_wgrad_accumulation=True)
    assert case["s"].calls == ["fwd", "zero_pad_rows"]           # only the no_grad call ran


def test_strided_main_grad_is_accepted(case):
    _, _, dw32 = _refs(case)
    w = case["w"]
    E, N, K = w.shape
    big = torch.randn(E, 2 * N, K)
    before = big.clone()
    w.main_grad = big[:, N:, :]                                   # row stride K, expert stride 2NK
    cake_grouped_det_mm(case["x"], w, case["offs"], fuse_wgrad_accumulation=True).backward(case["dy"])
    assert _eq(big[:, :N], before[:, :N])
    assert _eq(big[:, N:].contiguous(), torch.from_numpy(oracle.accumulate_fp32(before[:, N:].numpy(), dw32)))


def test_main_grad_sharing_memory_refused_at_backward(case):
    w = case["w"]
    E, N, K = w.shape
    M = case["x"].shape[0]
    buf = torch.zeros(E * N * K * 4 + M * K * 2, dtype=torch.uint8)
    x = buf[:M * K * 2].view(torch.bfloat16).view(M, K)
    x.copy_(case["x"].detach())
    x.requires_grad_()
    w.main_grad = buf[M * K * 2 - 64:M * K * 2 - 64 + E * N * K * 4].view(torch.float32).view(E, N, K)
    y = cake_grouped_det_mm(x, w, case["offs"], fuse_wgrad_accumulation=True)
    with pytest.raises(ValueError, match="shares memory with x"):
        y.backward(case["dy"])


def test_deterministic_mode_changes_nothing(case):
    w = case["w"]
    w.main_grad = case["main_grad"].clone()
    y0 = cake_grouped_det_mm(case["x"], w, case["offs"], fuse_wgrad_accumulation=True)
    y0.backward(case["dy"])
    a = (y0.detach().clone(), w.main_grad.clone(), case["x"].grad.clone())
    w.main_grad = case["main_grad"].clone()
    case["x"].grad = None
    prev = torch.are_deterministic_algorithms_enabled()
    torch.use_deterministic_algorithms(True)
    try:
        y1 = cake_grouped_det_mm(case["x"], w, case["offs"], fuse_wgrad_accumulation=True)
        y1.backward(case["dy"])
    finally:
        torch.use_deterministic_algorithms(prev)
    for u, v in zip(a, (y1.detach(), w.main_grad, case["x"].grad)):
        assert _eq(u, v)
