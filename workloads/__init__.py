"""Seeded synthetic workloads for the ragged BF16 grouped GEMM.

This module only draws inputs: group sizes, packed activations ``X [M, K]``,
expert weights ``W [E, N, K]``, output gradients ``G [M, N]`` and an fp32
``main_grad [E, N, K]``.  It holds none of the grouped GEMM's arithmetic and is
the one piece shared by the oracle side (tests, CPU baseline) and the HIP side
(tests, benchmark).

Groups follow the convention of the Cake ragged BF16 grouped GEMM API page
(docs.flashinfer.ai, "Cake ragged BF16 grouped GEMM", introduction): groups are
consecutive row ranges of the packed activations, described by ``offs[E]`` of
cumulative end offsets, or by ``m_indptr[E + 1]`` with a leading zero.

Values: X and W are N(0, 1)/sqrt(K), G is N(0, 1), each drawn in fp32 and rounded
to bfloat16 by torch's conversion; main_grad is 1e-2 * N(0, 1) in fp32.  Each
tensor has its own seeded ``torch.Generator`` so that a tensor can be re-drawn
alone.  Group sizes come from numpy's PCG64 (``numpy.random.default_rng``).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

__all__ = ["Workload", "CONFIGS", "group_sizes", "offsets_from_sizes",
           "indptr_from_sizes", "make_inputs", "TENSOR_STREAMS"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    E: int
    K: int
    N: int
    M: int
    recipe: str
    description: str


# Expert counts and shapes of the five MoE routing workloads used for parity and
# measurement: a tiny ragged case, a Mixtral-style top-2 layer (8 experts,
# hidden 4096, ffn 14336), a fine-grained 64-expert layer, a skewed 128-expert
# layer and a heavy-tailed 256-expert accumulate stress case.
CONFIGS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 4, 256, 256, 512, "fixed",
                     "E=4 K=256 N=256 M=512, group sizes [0,1,200,311]"),
    "mixtral": Workload("mixtral", 8, 4096, 14336, 16384, "uniform",
                        "E=8 K=4096 N=14336 M=16384 (8192 tokens x top-2), multinomial over uniform experts"),
    "fine": Workload("fine", 64, 2048, 1536, 32768, "dirichlet",
                     "E=64 K=2048 N=1536 M=32768, multinomial over Dirichlet(1) expert probabilities"),
    "skewed": Workload("skewed", 128, 7168, 4096, 32768, "zipf1.2",
                       "E=128 K=7168 N=4096 M=32768, Zipf(1.2) rank weights, ranks 119-128 at zero"),
    "stress": Workload("stress", 256, 7168, 2048, 65536, "zipf1.5",
                       "E=256 K=7168 N=2048 M=65536, Zipf(1.5) rank weights over all ranks"),
}

# The two MoE expert projections whose sizes flashinfer PR #8924 ("Cost") tabulates,
# at E = 4, 8, 16 and 32: gate_up (N=4096, K=6144) and down (N=6144, K=2048).  The
# pages give no token count; these use 8192 tokens routed top-2 (M = 16384 rows),
# multinomial over uniform experts, like the Mixtral-style case.
for _E in (4, 8, 16, 32):
    CONFIGS[f"gate_up_e{_E}"] = Workload(
        f"gate_up_e{_E}", _E, 6144, 4096, 16384, "uniform",
        f"gate_up projection E={_E} K=6144 N=4096 M=16384 (8192 tokens x top-2), uniform experts")
    CONFIGS[f"down_e{_E}"] = Workload(
        f"down_e{_E}", _E, 2048, 6144, 16384, "uniform",
        f"down projection E={_E} K=2048 N=6144 M=16384 (8192 tokens x top-2), uniform experts")
del _E

# Stream ids of the per-tensor generators: seed * 16 + id.
TENSOR_STREAMS = {"x": 1, "w": 2, "g": 3, "main_grad": 4}


def _zipf_sizes(rng: np.random.Generator, E: int, M: int, s: float, zero_ranks: int) -> np.ndarray:
    perm = rng.permutation(E)
    ranks = np.arange(1, E + 1, dtype=np.float64)
    weight = ranks ** (-s)
    if zero_ranks:
        weight[E - zero_ranks:] = 0.0
    p = np.zeros(E, dtype=np.float64)
    p[perm] = weight / weight.sum()
    return rng.multinomial(M, p)


def group_sizes(name: str, seed: int = 0) -> np.ndarray:
    """Rows per expert (int64 [E], summing to M) for a named workload."""
    cfg = CONFIGS[name]
    if cfg.recipe == "fixed":
        sizes = np.array([0, 1, 200, 311], dtype=np.int64)
    else:
        rng = np.random.default_rng(seed)
        if cfg.recipe == "uniform":
            sizes = rng.multinomial(cfg.M, [1.0 / cfg.E] * cfg.E)
        elif cfg.recipe == "dirichlet":
            p = rng.dirichlet(np.ones(cfg.E))
            sizes = rng.multinomial(cfg.M, p)
        elif cfg.recipe == "zipf1.2":
            sizes = _zipf_sizes(rng, cfg.E, cfg.M, 1.2, 10)
        elif cfg.recipe == "zipf1.5":
            sizes = _zipf_sizes(rng, cfg.E, cfg.M, 1.5, 0)
        else:  # pragma: no cover
            raise ValueError(cfg.recipe)
    sizes = np.asarray(sizes, dtype=np.int64)
    assert sizes.shape == (cfg.E,) and int(sizes.sum()) == cfg.M
    return sizes


def offsets_from_sizes(sizes) -> np.ndarray:
    """Cumulative end offsets offs[E] (int32)."""
    return np.cumsum(np.asarray(sizes, dtype=np.int64)).astype(np.int32)


def indptr_from_sizes(sizes) -> np.ndarray:
    """m_indptr[E + 1] (int32) with a leading zero."""
    return np.concatenate([[0], np.cumsum(np.asarray(sizes, dtype=np.int64))]).astype(np.int32)


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 16 + stream)
    return g


def _randn_bf16(shape, scale: float, seed: int, stream: int, device) -> torch.Tensor:
    gen = _gen(seed, stream, device)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    if out.numel() == 0:  # e.g. no rows at all: nothing to draw
        return out
    # Draw in slabs along dim 0 so that the fp32 staging stays small.
    flat = out.view(shape[0], -1)
    per_row = flat.shape[1]
    slab = max(1, (1 << 26) // max(per_row, 1))
    for r0 in range(0, shape[0], slab):
        r1 = min(shape[0], r0 + slab)
        t = torch.randn((r1 - r0, per_row), generator=gen, device=device, dtype=torch.float32)
        if scale != 1.0:
            t.mul_(scale)
        flat[r0:r1].copy_(t)
    return out


def make_inputs(name: Optional[str] = None, *, seed: int = 0, device="cpu",
                sizes=None, E: Optional[int] = None, K: Optional[int] = None,
                N: Optional[int] = None, M: Optional[int] = None,
                tensors=("x", "w", "g"), extra_rows: int = 0) -> dict:
    """Draw a workload's tensors on ``device``.

    Either ``name`` picks one of ``CONFIGS`` (its seeded group sizes), or
    ``sizes`` together with ``K`` and ``N`` give a custom case.  ``extra_rows``
    appends rows past the last group (row padding, which belongs to no group).
    Returns a dict with ``sizes`` (numpy), ``offs`` / ``m_indptr`` (int32 tensors
    on ``device``), the requested bf16 tensors and, if asked, ``main_grad``.
    """
    if name is not None:
        cfg = CONFIGS[name]
        E, K, N = cfg.E, cfg.K, cfg.N
        if sizes is None:
            sizes = group_sizes(name, seed)
    sizes = np.asarray(sizes, dtype=np.int64)
    E = int(sizes.shape[0]) if E is None else E
    assert sizes.shape == (E,)
    M_groups = int(sizes.sum())
    M = M_groups + extra_rows if M is None else M
    assert M >= M_groups
    out = {"sizes": sizes, "E": E, "K": K, "N": N, "M": M, "seed": seed}
    out["offs"] = torch.from_numpy(offsets_from_sizes(sizes)).to(device)
    out["m_indptr"] = torch.from_numpy(indptr_from_sizes(sizes)).to(device)
    inv = 1.0 / math.sqrt(K)
    if "x" in tensors:
        out["x"] = _randn_bf16((M, K), inv, seed, TENSOR_STREAMS["x"], device)
    if "w" in tensors:
        out["w"] = _randn_bf16((E, N, K), inv, seed, TENSOR_STREAMS["w"], device)
    if "g" in tensors:
        out["g"] = _randn_bf16((M, N), 1.0, seed, TENSOR_STREAMS["g"], device)
    if "main_grad" in tensors:
        gen = _gen(seed, TENSOR_STREAMS["main_grad"], device)
        mg = torch.empty((E, N, K), dtype=torch.float32, device=device)
        for e in range(E):
            mg[e].copy_(torch.randn((N, K), generator=gen, device=device, dtype=torch.float32))
        mg.mul_(1e-2)
        out["main_grad"] = mg
    return out
