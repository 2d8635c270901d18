"""Bitwise contracts on the GPU: reruns, the fused accumulate and zero rows."""
import numpy as np
import pytest
import torch

import moe_ragged_bf16_amd as mdg
from workloads import make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _poison(t):
    if t.dtype == torch.bfloat16:
        t.view(torch.int16).random_(-32768, 32767)
    else:
        t.view(torch.int32).random_(-2**31, 2**31 - 1)


# The third case has at least 2048 rows per group on average, so the forward takes the
# schedule that loads its stages in pairs; K = 1000 ends in a partial stage.
@pytest.mark.parametrize("case", [dict(name="tiny"), dict(sizes=[0, 1000, 3000, 5, 0], N=256, K=320),
                                  dict(sizes=[4100, 0, 2900, 5300], N=520, K=1000)])
def test_reruns_bitwise_with_poisoned_outputs(case):
    d = make_inputs(seed=5, device=DEV, **({"name": case["name"]} if "name" in case else
                                            {"sizes": case["sizes"], "N": case["N"], "K": case["K"]}))
    M, N, K, E = d["M"], d["N"], d["K"], d["E"]
    first = None
    for it in range(10):
        y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
        dw32 = torch.empty((E, N, K), dtype=torch.float32, device=DEV)
        dw16 = torch.empty((E, N, K), dtype=torch.bfloat16, device=DEV)
        for t in (y, dx, dw32, dw16):
            _poison(t)
        mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"], out=y)
        mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"], out=dx)
        mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out=dw32)
        mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out=dw16)
        cur = [y.view(torch.int16).clone(), dx.view(torch.int16).clone(),
               dw32.view(torch.int32).clone(), dw16.view(torch.int16).clone()]
        if first is None:
            first = cur
        else:
            for a, b in zip(first, cur):
                assert torch.equal(a, b), it


def test_accumulate_equals_adding_own_dw():
    d = make_inputs(sizes=[0, 1000, 3000, 5, 0, 77], N=512, K=320, seed=9, device=DEV,
                    tensors=("x", "g", "main_grad"))
    mg0 = d["main_grad"]
    # plant -0.0 on an empty expert and on a used one
    mg0[0, :3, :5] = -0.0
    mg0[1, 7, 9] = -0.0
    dw = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)
    expect = mg0 + dw                      # AccumulateGrad of the det dW: one fp32 add
    outs = []
    for _ in range(3):
        mg = mg0.clone()
        mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out=mg, accumulate=True)
        outs.append(mg)
    for mg in outs:
        assert torch.equal(mg.view(torch.int32), expect.view(torch.int32))
    assert not torch.signbit(outs[0][0, :3, :5]).any()      # -0.0 + 0.0 = +0.0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_accumulate_all_groups_empty_with_padding_rows(dtype):
    """m_rows > 0 but every group empty (offs all 0, the rows are padding): the
    accumulate adds the zero dW like adding the library's own overwrite dW does,
    so -0.0 becomes +0.0 and every other value is unchanged.  (m_rows == 0, the
    pages' sum_m == 0, launches nothing: see the next test.)"""
    E, N, K, M = 3, 256, 64, 37
    d = make_inputs(sizes=[0, 0, 0], N=N, K=K, extra_rows=M, seed=8, device=DEV, tensors=("x", "g"))
    mg0 = torch.randn((E, N, K), device=DEV).to(dtype)
    mg0[0, 0, :7] = -0.0
    dw = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=dtype)
    expect = mg0.clone().add_(dw)
    mg = mg0.clone()
    mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out=mg, accumulate=True)
    torch.cuda.synchronize()
    iv = torch.int32 if dtype == torch.float32 else torch.int16
    assert torch.all(dw.view(iv) == 0)
    assert torch.equal(mg.view(iv), expect.view(iv))
    assert not torch.signbit(mg[0, 0, :7].float()).any()


def test_accumulate_zero_rows_leaves_out_unchanged():
    E, N, K = 3, 256, 64
    g = torch.empty((0, N), dtype=torch.bfloat16, device=DEV)
    x = torch.empty((0, K), dtype=torch.bfloat16, device=DEV)
    offs = torch.zeros(E, dtype=torch.int32, device=DEV)
    mg = torch.randn((E, N, K), device=DEV)
    mg[0, 0, 0] = -0.0
    before = mg.clone()
    mdg.grouped_det_gemm_wgrad(g, x, offs, out=mg, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(mg.view(torch.int32), before.view(torch.int32))
    # overwrite with zero rows writes +0.0
    dw = mdg.grouped_det_gemm_wgrad(g, x, offs, out_dtype=torch.float32)
    assert torch.all(dw.view(torch.int32) == 0)
    y = mdg.grouped_det_gemm_fwd(x, torch.zeros((E, N, K), dtype=torch.bfloat16, device=DEV), offs)
    assert y.shape == (0, N)


def test_offsets_rewritten_in_place_give_new_result():
    d = make_inputs(sizes=[100, 200, 300], N=256, K=128, seed=2, device=DEV)
    y1 = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"]).clone()
    d["offs"].copy_(torch.tensor([300, 300, 600], dtype=torch.int32, device=DEV))
    y2 = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    ref2 = (d["x"][:300].float() @ d["w"][0].float().T)
    torch.cuda.synchronize()
    assert not torch.equal(y1[100:300], y2[100:300])
    err = (y2[:300].float() - ref2).abs().max() / ref2.abs().max()
    assert err < 2e-2


def test_two_streams_same_bits():
    d = make_inputs(sizes=[500, 0, 900], N=512, K=256, seed=4, device=DEV)
    ref = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        a = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)
    with torch.cuda.stream(s2):
        b = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), ref.view(torch.int32))
    assert torch.equal(b.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("sizes", [[0, 1000, 3000, 5, 0, 77], [64, 0, 200]])
def test_accumulate_bf16_equals_adding_own_dw(sizes):
    """bf16 out: the bf16 overwrite dW added in bf16, bitwise (torch's bf16 add
    and the oracle's reading of it), run to run; split and unsplit experts."""
    d = make_inputs(sizes=sizes, N=512, K=320, seed=19, device=DEV, tensors=("x", "g", "main_grad"))
    print(f"bf16 accumulate: sizes={sizes}", flush=True)
    mg0 = d["main_grad"].to(torch.bfloat16)
    mg0[0, :3, :5] = -0.0
    dw = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out_dtype=torch.bfloat16)
    expect = mg0.clone().add_(dw)
    outs = []
    for _ in range(3):
        mg = mg0.clone()
        mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out=mg, accumulate=True)
        outs.append(mg)
    for mg in outs:
        assert torch.equal(mg.view(torch.int16), expect.view(torch.int16))
    from _parity import bits
    import oracle
    assert np.array_equal(bits(outs[0]), oracle.accumulate_bf16(bits(mg0), bits(dw)))


def test_accumulate_bf16_zero_rows_leaves_out_unchanged():
    E, N, K = 3, 256, 64
    g = torch.empty((0, N), dtype=torch.bfloat16, device=DEV)
    x = torch.empty((0, K), dtype=torch.bfloat16, device=DEV)
    offs = torch.zeros(E, dtype=torch.int32, device=DEV)
    mg = torch.randn((E, N, K), device=DEV).to(torch.bfloat16)
    mg[0, 0, 0] = -0.0
    before = mg.clone()
    mdg.grouped_det_gemm_wgrad(g, x, offs, out=mg, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(mg.view(torch.int16), before.view(torch.int16))


@pytest.mark.parametrize("dtype,cols", [(torch.bfloat16, 256), (torch.float32, 64), (torch.bfloat16, 8)])
def test_zero_pad_rows(dtype, cols):
    M, E = 1000, 4
    for ends in ([100, 300, 300, 777], [0, 0, 0, 0], [10, 20, 30, 1000], [5, 6, 7, 4000], [5, 6, 7, -3]):
        out = torch.randn((M, cols), device=DEV).to(dtype)
        before = out.clone()
        offs = torch.tensor(ends, dtype=torch.int32, device=DEV)
        mdg.zero_pad_rows(out, offs, E)
        t = min(max(max(ends), 0), M)   # the last end the GEMMs use: the largest clamped offset
        torch.cuda.synchronize()
        assert torch.equal(out[:t], before[:t]), ends
        assert torch.all(out[t:] == 0) and not torch.signbit(out[t:].float()).any(), ends
    # the m_indptr form gives the same last end
    out = torch.ones((M, cols), device=DEV).to(dtype)
    mdg.zero_pad_rows(out, torch.tensor([0, 10, 20, 30, 500], dtype=torch.int32, device=DEV), E)
    assert torch.all(out[:500] == 1) and torch.all(out[500:] == 0)
    # no rows: nothing to do
    mdg.zero_pad_rows(torch.empty((0, cols), dtype=dtype, device=DEV), offs, E)


def test_inference_tensors():
    """Inference-mode tensors as inputs and as the accumulate target (they have
    no version counter): same bits as ordinary tensors."""
    d = make_inputs(sizes=[300, 0, 700], N=256, K=192, seed=25, device=DEV, tensors=("x", "w", "g", "main_grad"))
    y0 = mdg.grouped_det_gemm_fwd(d["x"], d["w"], d["offs"])
    mg0 = d["main_grad"].clone()
    mdg.grouped_det_gemm_wgrad(d["g"], d["x"], d["offs"], out=mg0, accumulate=True)
    with torch.inference_mode():
        x, w, g = d["x"].clone(), d["w"].clone(), d["g"].clone()
        offs = d["offs"].clone()
        mg = d["main_grad"].clone()
        assert x.is_inference() and mg.is_inference()
        y = mdg.grouped_det_gemm_fwd(x, w, offs)
        mdg.grouped_det_gemm_wgrad(g, x, offs, out=mg, accumulate=True)
        l = mdg.prepare_grouped_det_gemm_dgrad(g, w, offs)
        dx = l.launch()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y0.view(torch.int16))
    assert torch.equal(mg.view(torch.int32), mg0.view(torch.int32))
    assert torch.equal(dx[:1000].view(torch.int16),
                       mdg.grouped_det_gemm_dgrad(d["g"], d["w"], d["offs"])[:1000].view(torch.int16))


@pytest.mark.parametrize("bad", [
    [-5, 700, 300, 5000, 2000],      # negative, decreasing, past m_rows
    [2**31 - 1] * 5,                 # all past m_rows: group 0 takes every row
    [-2**31, -1, 0, -7, 2900],       # negatives
])
def test_malformed_offsets_act_as_clamped(bad):
    """The kernels clamp each offset to [0, m_rows] and take the running maximum, so a
    malformed array reads and writes nothing out of bounds and gives, bit for bit, the
    result of its sanitised form, the zero fill of the padding rows included.  Every
    host-side size depends on m_rows and the group count only, which any sanitised
    array respects."""
    M, N, K = 3000, 520, 328
    d = make_inputs(sizes=[600] * 5, N=N, K=K, seed=21, device=DEV, tensors=("x", "w", "g", "main_grad"))
    clean = np.maximum.accumulate(np.clip(np.asarray(bad, dtype=np.int64), 0, M))

    def run(offs):
        y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
        dx = torch.full((M, K), 7.0, dtype=torch.bfloat16, device=DEV)
        mdg.grouped_det_gemm_fwd(d["x"], d["w"], offs, out=y)
        mdg.grouped_det_gemm_dgrad(d["g"], d["w"], offs, out=dx)
        dw = mdg.grouped_det_gemm_wgrad(d["g"], d["x"], offs, out_dtype=torch.float32)
        mg = d["main_grad"].clone()
        mdg.grouped_det_gemm_wgrad(d["g"], d["x"], offs, out=mg, accumulate=True)
        z = torch.full((M, 64), 7.0, dtype=torch.bfloat16, device=DEV)
        mdg.zero_pad_rows(z, offs, 5)
        torch.cuda.synchronize()
        return [y.view(torch.int16), dx.view(torch.int16), dw.view(torch.int32), mg.view(torch.int32),
                z.view(torch.int16)]

    got = run(torch.tensor(bad, dtype=torch.int32, device=DEV))
    want = run(torch.tensor(clean, dtype=torch.int32, device=DEV))
    for a, b in zip(got, want):
        assert torch.equal(a, b)
    # the sanitised groups: empty ones give exactly zero dW, rows past the last end stay untouched
    sizes = np.diff(np.concatenate([[0], clean]))
    for e in np.flatnonzero(sizes == 0):
        assert torch.all(got[2][e] == 0)
    seven = torch.tensor(7.0, dtype=torch.bfloat16).view(torch.int16).item()
    if clean[-1] < M:
        assert torch.all(got[0][clean[-1]:] == seven)
    # the zero fill covers exactly the rows past the sanitised last end
    assert torch.all(got[4][:clean[-1]] == seven) and torch.all(got[4][clean[-1]:] == 0)
