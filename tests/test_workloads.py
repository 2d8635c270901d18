"""The seeded workload generators meet the properties each workload states."""
import numpy as np
import pytest
import torch

from workloads import CONFIGS, group_sizes, indptr_from_sizes, make_inputs, offsets_from_sizes


@pytest.mark.parametrize("name", list(CONFIGS))
def test_sizes_sum_and_reproducible(name):
    cfg = CONFIGS[name]
    a = group_sizes(name, 0)
    b = group_sizes(name, 0)
    assert a.shape == (cfg.E,) and int(a.sum()) == cfg.M and (a >= 0).all()
    np.testing.assert_array_equal(a, b)


def test_tiny_sizes():
    s = group_sizes("tiny")
    np.testing.assert_array_equal(s, [0, 1, 200, 311])
    np.testing.assert_array_equal(offsets_from_sizes(s), [0, 1, 201, 512])
    np.testing.assert_array_equal(indptr_from_sizes(s), [0, 0, 1, 201, 512])


def test_mixtral_sizes():
    s = group_sizes("mixtral")
    assert s.min() > 1900 and s.max() < 2200       # near-uniform over 8 experts


def test_fine_sizes():
    s = group_sizes("fine")
    assert (s == 0).sum() >= 1                      # some group is empty
    assert ((s > 0) & (s < 64)).sum() >= 4          # several tiny groups
    assert s.max() > 4 * np.median(s)               # Dirichlet(1) is uneven


def test_skewed_sizes():
    s = group_sizes("skewed")
    assert (s == 0).sum() >= 10                     # at least ten empty groups
    assert s.max() > 4000                           # one dominant group
    assert ((s % 64) != 0).sum() >= 100             # mostly not tile multiples


def test_stress_sizes():
    s = group_sizes("stress")
    assert s.max() > 20000 and np.median(s) < 64    # heavy tail
    assert ((s % 64) != 0).sum() > 200              # mostly non-multiples of 64


def test_make_inputs_tiny_shapes_and_determinism():
    a = make_inputs("tiny", seed=0, tensors=("x", "w", "g", "main_grad"))
    b = make_inputs("tiny", seed=0, tensors=("x", "w", "g", "main_grad"))
    assert a["x"].shape == (512, 256) and a["x"].dtype == torch.bfloat16
    assert a["w"].shape == (4, 256, 256) and a["g"].shape == (512, 256)
    assert a["main_grad"].shape == (4, 256, 256) and a["main_grad"].dtype == torch.float32
    for k in ("x", "w", "g", "main_grad"):
        assert torch.equal(a[k], b[k])
    c = make_inputs("tiny", seed=1)
    assert not torch.equal(a["x"], c["x"])
    # scales: X, W ~ N(0,1)/sqrt(K); G ~ N(0,1); main_grad ~ 1e-2 N(0,1)
    assert abs(a["x"].float().std().item() - 1 / 16) < 0.01
    assert abs(a["g"].float().std().item() - 1.0) < 0.05
    assert abs(a["main_grad"].std().item() - 1e-2) < 1e-3


def test_make_inputs_custom_and_padding():
    d = make_inputs(sizes=[3, 0, 5], K=64, N=256, extra_rows=4)
    assert d["M"] == 12 and d["x"].shape == (12, 64)
    assert d["offs"].tolist() == [3, 3, 8] and d["m_indptr"].tolist() == [0, 3, 3, 8]


def test_make_inputs_without_rows():
    """Every group empty and no padding: zero-row tensors, offsets all zero."""
    d = make_inputs(sizes=[0, 0, 0], N=256, K=64, seed=1, tensors=("x", "w", "g", "main_grad"))
    assert d["M"] == 0 and d["x"].shape == (0, 64) and d["g"].shape == (0, 256)
    assert d["w"].shape == (3, 256, 64) and d["offs"].tolist() == [0, 0, 0]
