"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: a hand-worked example
(tests/golden/hand_worked_small.json), hand-derived rounding cases
(tests/golden/rounding_cases.json), a pure-Python fp64 brute force on tiny
inputs, closed forms with one-hot operands, and invariants (adjoint identity,
empty groups, permutation of experts, regrouping).  A dropped term, a wrong
sign or index, a transposed operand or a wrong group boundary in the oracle
fails at least one of these.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits_of(values) -> np.ndarray:
    """bf16 bit patterns of values that are exact in bf16 (via torch's conversion)."""
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _np_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _rand_bits(rng, shape, scale=1.0):
    v = (rng.standard_normal(shape) * scale).astype(np.float32)
    return _bits_of(v)


# ---------------------------------------------------------------- golden example
@pytest.fixture(scope="module")
def hand():
    with open(os.path.join(GOLDEN, "hand_worked_small.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("precision", ["fp64", "fp32"])
def test_hand_example_fwd_dgrad_wgrad(hand, precision):
    X, W, G = (_bits_of(hand[k]) for k in ("X", "W", "G"))
    offs = np.array(hand["offs"], dtype=np.int32)
    y = oracle.fwd(X, W, offs, precision)
    dx = oracle.dgrad(G, W, offs, precision)
    dw = oracle.wgrad(G, X, offs, precision)
    np.testing.assert_array_equal(y[:3], np.array(hand["Y_rows_0_to_2"]))
    np.testing.assert_array_equal(dx[:3], np.array(hand["dX_rows_0_to_2"]))
    np.testing.assert_array_equal(dw, np.array(hand["dW"]))
    # the padding row (past offs[E-1]) belongs to no group
    assert np.all(np.isnan(y[3])) and np.all(np.isnan(dx[3]))
    # the empty group's dW is +0.0 in every bit
    assert not np.any(np.signbit(dw[1]))


def test_hand_example_indptr_form(hand):
    offs = oracle.offs_from_indptr(np.array(hand["m_indptr"], dtype=np.int32))
    np.testing.assert_array_equal(offs, hand["offs"])
    with pytest.raises(ValueError):
        oracle.offs_from_indptr(np.array([1, 2, 3]))


def test_hand_example_adjoint(hand):
    X, W, G = (_bits_of(hand[k]) for k in ("X", "W", "G"))
    offs = np.array(hand["offs"], dtype=np.int32)
    y = oracle.fwd(X, W, offs)[:3]
    dx = oracle.dgrad(G, W, offs)[:3]
    dw = oracle.wgrad(G, X, offs)
    g = oracle.widen_bf16(G)[:3].astype(np.float64)
    x = oracle.widen_bf16(X)[:3].astype(np.float64)
    w = oracle.widen_bf16(W).astype(np.float64)
    target = hand["adjoint_inner_product"]
    assert np.sum(y * g) == target
    assert np.sum(x * dx) == target
    assert np.sum(w * dw) == target


# ---------------------------------------------------------------- brute force
def _brute(Xf, Wf, Gf, offs):
    """Pure-Python fp64 triple loops straight from the operations table."""
    M, K = len(Xf), len(Xf[0])
    E, N = len(Wf), len(Wf[0])
    Y = [[None] * N for _ in range(M)]
    dX = [[None] * K for _ in range(M)]
    dW = [[[0.0] * K for _ in range(N)] for _ in range(E)]
    start = 0
    for e in range(E):
        end = int(offs[e])
        for i in range(start, end):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    acc += float(Xf[i][k]) * float(Wf[e][n][k])
                Y[i][n] = acc
            for k in range(K):
                acc = 0.0
                for n in range(N):
                    acc += float(Gf[i][n]) * float(Wf[e][n][k])
                dX[i][k] = acc
        for n in range(N):
            for k in range(K):
                acc = 0.0
                for i in range(start, end):
                    acc += float(Gf[i][n]) * float(Xf[i][k])
                dW[e][n][k] = acc
        start = end
    return Y, dX, dW


@pytest.mark.parametrize("sizes,N,K,pad", [
    ([3], 4, 5, 0),
    ([0, 2, 1], 3, 7, 0),
    ([1, 0, 0, 4], 5, 3, 2),
    ([2, 5], 6, 4, 1),
    ([0, 0], 2, 2, 3),
])
@pytest.mark.parametrize("precision,tol", [("fp64", 1e-12), ("fp32", 1e-5)])
def test_bruteforce_micro(sizes, N, K, pad, precision, tol):
    rng = np.random.default_rng(sum(sizes) * 131 + N * 7 + K)
    E = len(sizes)
    M = sum(sizes) + pad
    X = _rand_bits(rng, (M, K))
    W = _rand_bits(rng, (E, N, K))
    G = _rand_bits(rng, (M, N))
    offs = np.cumsum(sizes).astype(np.int32)
    Xf, Wf, Gf = (oracle.widen_bf16(a).tolist() for a in (X, W, G))
    Yb, dXb, dWb = _brute(Xf, Wf, Gf, offs)
    y = oracle.fwd(X, W, offs, precision)
    dx = oracle.dgrad(G, W, offs, precision)
    dw = oracle.wgrad(G, X, offs, precision)
    Mg = int(offs[-1]) if E else 0
    Yb_a = np.array(Yb[:Mg], dtype=np.float64).reshape(Mg, N)
    dXb_a = np.array(dXb[:Mg], dtype=np.float64).reshape(Mg, K)
    dWb_a = np.array(dWb, dtype=np.float64)
    scale = max(1.0, float(np.abs(Yb_a).max(initial=0)), float(np.abs(dXb_a).max(initial=0)),
                float(np.abs(dWb_a).max(initial=0)))
    assert np.max(np.abs(y[:Mg] - Yb_a), initial=0) <= tol * scale
    assert np.max(np.abs(dx[:Mg] - dXb_a), initial=0) <= tol * scale
    assert np.max(np.abs(dw - dWb_a), initial=0) <= tol * scale
    assert np.all(np.isnan(y[Mg:])) and np.all(np.isnan(dx[Mg:]))
    for e, m in enumerate(sizes):
        if m == 0:
            assert np.all(dw[e] == 0) and not np.any(np.signbit(dw[e]))


# ---------------------------------------------------------------- closed forms
def test_one_hot_closed_forms():
    """One-hot rows pick single entries of W: Y[i, n] = W[e, n, k(i)],
    dX[i, k] = W[e, n(i), k] and dW[e] counts the (n(i), k(i)) pairs."""
    rng = np.random.default_rng(7)
    E, N, K = 3, 6, 5
    sizes = [4, 0, 3]
    M = sum(sizes)
    offs = np.cumsum(sizes).astype(np.int32)
    kk = rng.integers(0, K, M)
    nn = rng.integers(0, N, M)
    Xv = np.zeros((M, K), np.float32)
    Xv[np.arange(M), kk] = 1.0
    Gv = np.zeros((M, N), np.float32)
    Gv[np.arange(M), nn] = 1.0
    Wv = np.round(rng.standard_normal((E, N, K)) * 8).astype(np.float32)
    X, G, W = _bits_of(Xv), _bits_of(Gv), _bits_of(Wv)
    y = oracle.fwd(X, W, offs)
    dx = oracle.dgrad(G, W, offs)
    dw = oracle.wgrad(G, X, offs)
    expert = np.repeat(np.arange(E), sizes)
    for i in range(M):
        e = expert[i]
        np.testing.assert_array_equal(y[i], Wv[e, :, kk[i]])
        np.testing.assert_array_equal(dx[i], Wv[e, nn[i], :])
    for e in range(E):
        cnt = np.zeros((N, K))
        for i in np.nonzero(expert == e)[0]:
            cnt[nn[i], kk[i]] += 1
        np.testing.assert_array_equal(dw[e], cnt)


# ---------------------------------------------------------------- invariants
@pytest.fixture(scope="module")
def tiny():
    d = make_inputs("tiny", seed=0, device="cpu")
    return {"X": _np_bits(d["x"]), "W": _np_bits(d["w"]), "G": _np_bits(d["g"]),
            "offs": d["offs"].numpy(), "sizes": d["sizes"]}


def test_adjoint_identity_tiny(tiny):
    X, W, G, offs = tiny["X"], tiny["W"], tiny["G"], tiny["offs"]
    y, dx, dw = oracle.fwd(X, W, offs), oracle.dgrad(G, W, offs), oracle.wgrad(G, X, offs)
    a = np.sum(y * oracle.widen_bf16(G))
    b = np.sum(dx * oracle.widen_bf16(X))
    c = np.sum(dw * oracle.widen_bf16(W))
    scale = np.sum(np.abs(y * oracle.widen_bf16(G)))
    assert abs(a - b) <= 1e-12 * scale and abs(a - c) <= 1e-12 * scale


def test_empty_group_exact_zero_tiny(tiny):
    dw = oracle.wgrad(tiny["G"], tiny["X"], tiny["offs"], "fp32")
    assert tiny["sizes"][0] == 0
    assert np.all(dw[0].view(np.uint32) == 0)


def test_fp32_matches_fp64_tiny(tiny):
    X, W, G, offs = tiny["X"], tiny["W"], tiny["G"], tiny["offs"]
    for f in (lambda p: oracle.fwd(X, W, offs, p), lambda p: oracle.dgrad(G, W, offs, p),
              lambda p: oracle.wgrad(G, X, offs, p)):
        a, b = f("fp32"), f("fp64")
        m = ~np.isnan(b)
        assert np.max(np.abs(a[m] - b[m])) <= 1e-5 * np.max(np.abs(b[m]))


def test_permuting_experts_permutes_outputs(tiny):
    X, W, G, sizes = tiny["X"], tiny["W"], tiny["G"], tiny["sizes"]
    perm = np.array([2, 0, 3, 1])
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    rows = np.concatenate([np.arange(starts[e], starts[e] + sizes[e]) for e in perm]).astype(np.int64)
    offs2 = np.cumsum(sizes[perm]).astype(np.int32)
    y1 = oracle.fwd(X, W, tiny["offs"])
    y2 = oracle.fwd(X[rows], W[perm], offs2)
    np.testing.assert_array_equal(y2, y1[rows])
    dx2 = oracle.dgrad(G[rows], W[perm], offs2)
    np.testing.assert_array_equal(dx2, oracle.dgrad(G, W, tiny["offs"])[rows])
    dw2 = oracle.wgrad(G[rows], X[rows], offs2)
    np.testing.assert_allclose(dw2, oracle.wgrad(G, X, tiny["offs"])[perm], rtol=0, atol=1e-12)


def test_regrouping_with_shared_weight(tiny):
    """Splitting group 3 into two groups with the same weight leaves Y/dX
    unchanged and splits dW into two parts that sum to the original."""
    X, W, G, sizes = tiny["X"], tiny["W"], tiny["G"], tiny["sizes"]
    offs = tiny["offs"]
    split = 100
    offs2 = np.array(list(offs[:3]) + [offs[2] + split, offs[3]], dtype=np.int32)
    W2 = np.concatenate([W, W[3:4]], axis=0)
    np.testing.assert_array_equal(oracle.fwd(X, W2, offs2), oracle.fwd(X, W, offs))
    np.testing.assert_array_equal(oracle.dgrad(G, W2, offs2), oracle.dgrad(G, W, offs))
    dw = oracle.wgrad(G, X, offs)
    dw2 = oracle.wgrad(G, X, offs2)
    np.testing.assert_allclose(dw2[3] + dw2[4], dw[3], rtol=0, atol=1e-12)


def test_sampled_forms_match_full(tiny):
    X, W, G, offs = tiny["X"], tiny["W"], tiny["G"], tiny["offs"]
    rows = np.array([0, 1, 5, 200, 201, 511])
    np.testing.assert_array_equal(oracle.fwd_rows(X, W, offs, rows), oracle.fwd(X, W, offs)[rows])
    np.testing.assert_array_equal(oracle.dgrad_rows(G, W, offs, rows), oracle.dgrad(G, W, offs)[rows])
    dw = oracle.wgrad(G, X, offs)
    np.testing.assert_array_equal(oracle.wgrad_expert(G[201:512], X[201:512]), dw[3])
    np.testing.assert_array_equal(oracle.wgrad_expert(G[0:0], X[0:0]), dw[0])


def test_group_ranges_rejects_bad_offsets():
    with pytest.raises(ValueError):
        oracle.group_ranges([3, 2], 5)      # decreasing
    with pytest.raises(ValueError):
        oracle.group_ranges([2, 6], 5)      # past the rows
    with pytest.raises(ValueError):
        oracle.group_ranges([-1, 2], 5)     # negative
    assert oracle.group_ranges([0, 0, 5], 5) == [(0, 0), (0, 0), (0, 5)]
    with pytest.raises(ValueError):
        oracle.fwd_rows(*(np.zeros((4, 2), np.uint16), np.zeros((1, 2, 2), np.uint16)),
                        [2], [3])           # row 3 is padding


# ---------------------------------------------------------------- rounding
@pytest.fixture(scope="module")
def rounding():
    with open(os.path.join(GOLDEN, "rounding_cases.json")) as f:
        return json.load(f)


def test_bf16_rne_hand_cases(rounding):
    for c in rounding["bf16_rne"]:
        f = np.array([int(c["f32_bits"], 16)], dtype=np.uint32).view(np.float32)
        assert int(oracle.round_bf16_rne(f)[0]) == int(c["bf16_bits"], 16), c["why"]


def test_bf16_rne_nan():
    for bits in (0x7FC00000, 0x7F800001, 0xFFFFFFFF, 0x7F80FFFF):
        f = np.array([bits], dtype=np.uint32).view(np.float32)
        r = oracle.round_bf16_rne(f)
        assert np.isnan(oracle.widen_bf16(r))[0]


def test_bf16_rne_matches_torch_on_random_bits():
    """torch's fp32 -> bf16 conversion is an independent RNE implementation."""
    rng = np.random.default_rng(3)
    u = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[~np.isnan(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.round_bf16_rne(f), ref)


def test_widen_bf16_matches_torch_and_definition():
    b = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    w = oracle.widen_bf16(b)
    t = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    same = (w.view(np.uint32) == t.view(np.uint32)) | (np.isnan(w) & np.isnan(t))
    assert same.all()
    assert oracle.widen_bf16(np.array([0x3F80], np.uint16))[0] == 1.0
    assert oracle.widen_bf16(np.array([0xC040], np.uint16))[0] == -3.0


def test_accumulate_fp32_hand_cases(rounding):
    for c in rounding["fp32_add"]:
        a = np.array([int(c["a"], 16)], np.uint32).view(np.float32)
        b = np.array([int(c["b"], 16)], np.uint32).view(np.float32)
        r = oracle.accumulate_fp32(a, b)
        assert int(r.view(np.uint32)[0]) == int(c["sum"], 16), c["why"]


def test_accumulate_fp32_is_single_rounding_of_exact_sum():
    """RN32(a + b): the exact sum (fp64 holds it for fp32 inputs within range)
    rounded once to fp32."""
    rng = np.random.default_rng(11)
    a = (rng.standard_normal(100000) * 1e-2).astype(np.float32)
    b = (rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 2, 100000)).astype(np.float32)
    exact = a.astype(np.float64) + b.astype(np.float64)
    np.testing.assert_array_equal(oracle.accumulate_fp32(a, b).view(np.uint32),
                                  exact.astype(np.float32).view(np.uint32))


def test_accumulate_bf16_matches_torch_bf16_add():
    rng = np.random.default_rng(5)
    a = _rand_bits(rng, (50000,), 1.0)
    b = _rand_bits(rng, (50000,), 1e-2)
    ta = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    tb = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16)
    ref = (ta + tb).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.accumulate_bf16(a, b), ref)
