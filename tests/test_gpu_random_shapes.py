"""Seeded random shapes on the GPU against the oracle: expert counts 1-12, N and K
multiples of 8 up to 1024 / 768 (partial 256-wide tiles in every direction and
reductions that end in a partial 32-deep stage),
group sizes drawn four ways (uniform, Dirichlet-skewed, tile-boundary values,
mostly empty), padding rows; every output element of fwd, dgrad and wgrad (bf16
and fp32) against the fp64 oracle, and both accumulate dtypes bitwise against
adding the library's own dW."""
import numpy as np
import pytest
import torch

import moe_ragged_bf16_amd as mdg
from workloads import make_inputs
from test_gpu_parity import _check_full

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _shape(seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.integers(1, 13))
    N = 8 * int(rng.integers(1, 129))
    K = 8 * int(rng.integers(1, 97))
    kind = seed % 4
    if kind == 0:
        sizes = rng.integers(0, 400, E)
    elif kind == 1:
        sizes = rng.multinomial(int(rng.integers(0, 3000)), rng.dirichlet(np.full(E, 0.3)))
    elif kind == 2:
        sizes = rng.choice([0, 1, 31, 32, 33, 255, 256, 257, 511, 512, 513], E)
    else:
        sizes = rng.integers(0, 2, E) * rng.integers(1, 1500, E)
    return np.asarray(sizes, dtype=np.int64), N, K, int(rng.integers(0, 6))


@pytest.mark.parametrize("seed", range(24))
def test_random_shape(seed):
    sizes, N, K, pad = _shape(seed)
    label = f"seed={seed} sizes={sizes.tolist()} N={N} K={K} pad={pad}"
    print(label, flush=True)
    d = make_inputs(sizes=sizes, N=N, K=K, extra_rows=pad, seed=seed, device=DEV,
                    tensors=("x", "w", "g", "main_grad"))
    _check_full(d, label)
    for dt in (torch.float32, torch.bfloat16):
        mg0 = d["main_grad"].to(dt)
        mg = mg0.clone()
        mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out=mg, accumulate=True)
        dw = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=dt)
        v = torch.int32 if dt == torch.float32 else torch.int16
        assert torch.equal(mg.view(v), mg0.add_(dw).view(v)), (label, dt)
