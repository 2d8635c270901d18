"""Seeded random shapes between the small random cases and the full workloads:
N and K multiples of 8 up to 4096 (long reductions ending in partial stages and
partial tiles in both directions), 1-64 experts, up to 16k rows in Dirichlet,
uniform or Zipf-like groups, padding rows.  Every output element of fwd, dgrad
and wgrad (fp32 and bf16) against the fp32 CPU oracle expert by expert (the
same gates as everywhere: max |gpu - ref| / max |ref| per group <= 2e-2 for bf16
outputs, 1e-3 for fp32 dW), empty experts exactly zero dW, and the fused fp32
accumulate bitwise equal to adding the library's own dW."""
import numpy as np
import pytest
import torch

import moe_ragged_bf16_amd as mdg
import oracle
from workloads import make_inputs
from _parity import TOL_BF16, TOL_FP32, bits, ranges

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _f32(t):
    return oracle.widen_bf16(bits(t)) if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def _err(gpu, ref):
    diff = float(np.max(np.abs(gpu - ref)))
    scale = float(np.max(np.abs(ref)))
    return diff / scale if scale > 0 else (0.0 if diff == 0 else float("inf"))


def _shape(seed):
    rng = np.random.default_rng(40000 + seed)
    E = int(rng.integers(1, 65))
    N = 8 * int(rng.integers(1, 513))
    K = 8 * int(rng.integers(1, 513))
    M = int(rng.integers(0, 16385))
    while M * N * K > (1 << 36):     # keeps the CPU oracle to a fraction of a second per op
        M //= 2
    kind = seed % 3
    if kind == 0:
        sizes = rng.multinomial(M, rng.dirichlet(np.full(E, 0.3)))
    elif kind == 1:
        sizes = rng.multinomial(M, np.full(E, 1.0 / E))
    else:
        w = np.arange(1, E + 1, dtype=np.float64) ** -1.3
        rng.shuffle(w)
        sizes = rng.multinomial(M, w / w.sum())
    return np.asarray(sizes, dtype=np.int64), N, K, int(rng.integers(0, 11))


@pytest.mark.parametrize("seed", range(10))
def test_mid_shape(seed):
    sizes, N, K, pad = _shape(seed)
    label = f"seed={seed} E={len(sizes)} N={N} K={K} M={int(sizes.sum())} pad={pad}"
    print(label, flush=True)
    d = make_inputs(sizes=sizes, N=N, K=K, extra_rows=pad, seed=seed, device=DEV,
                    tensors=("x", "w", "g", "main_grad"))
    y = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    dx = mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"])
    dw32 = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)
    dw16 = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.bfloat16)
    mg = d["main_grad"].clone()
    mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out=mg, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(mg.view(torch.int32), d["main_grad"].clone().add_(dw32).view(torch.int32)), label
    one = np.array([0], dtype=np.int32)
    for e, (s, t) in enumerate(ranges(sizes)):
        if t == s:
            assert torch.all(dw32[e].view(torch.int32) == 0) and torch.all(dw16[e].view(torch.int16) == 0), (label, e)
            continue
        one[0] = t - s
        X, G, W = bits(d["x"][s:t]), bits(d["g"][s:t]), bits(d["w"][e:e + 1])
        assert _err(_f32(y[s:t]), oracle.fwd(X, W, one, precision="fp32")) <= TOL_BF16, (label, "fwd", e)
        assert _err(_f32(dx[s:t]), oracle.dgrad(G, W, one, precision="fp32")) <= TOL_BF16, (label, "dgrad", e)
        ref = oracle.wgrad_expert(G, X, precision="fp32")
        assert _err(_f32(dw32[e]), ref) <= TOL_FP32, (label, "wgrad fp32", e)
        assert _err(_f32(dw16[e]), ref) <= TOL_BF16, (label, "wgrad bf16", e)
