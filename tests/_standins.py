"""CPU stand-ins for the device entry points, built on the oracle (test
infrastructure only).

They keep the binding's contracts that the autograd wrapper relies on: outputs
are fresh tensors unless ``out`` is given, rows past offs[E-1] of a fresh fwd /
dgrad output are left unwritten (NaN here, so a missing fill shows), wgrad can
add into ``out`` with the bits of ``out.add_(dW)`` in out's dtype, and a
written ``out`` gets its version counter bumped.  Installed with
``install(monkeypatch)``; ``calls`` records each entry's name.
"""
import numpy as np
import torch

import oracle


def _bits(t):
    return t.detach().contiguous().view(torch.int16).numpy().view(np.uint16)


def _bf16(a32):
    return torch.from_numpy(oracle.round_bf16_rne(np.asarray(a32, dtype=np.float32)).view(np.int16)) \
        .view(torch.bfloat16)


def _offs(offs, E):
    o = offs.cpu().numpy().astype(np.int64)
    return oracle.offs_from_indptr(o) if o.shape[0] == E + 1 else o


class StandIns:
    def __init__(self):
        self.calls = []

    def fwd(self, x, w, offs, out=None, workspace=None):
        self.calls.append("fwd")
        y = oracle.fwd(_bits(x), _bits(w), _offs(offs, w.shape[0]), precision="fp32")
        return _bf16(y)

    def dgrad(self, g, w, offs, out=None, workspace=None):
        self.calls.append("dgrad")
        dx = oracle.dgrad(_bits(g), _bits(w), _offs(offs, w.shape[0]), precision="fp32")
        return _bf16(dx)

    def wgrad(self, g, x, offs, out=None, out_dtype=None, num_groups=None, *, accumulate=False,
              workspace=None):
        self.calls.append("wgrad_acc" if accumulate else "wgrad")
        E = out.shape[0] if out is not None else (num_groups if num_groups is not None else offs.numel())
        dw32 = oracle.wgrad(_bits(g), _bits(x), _offs(offs, E), precision="fp32").astype(np.float32)
        dt = out.dtype if out is not None else (out_dtype or torch.bfloat16)
        assert out is None or out.is_contiguous()
        if dt == torch.float32:
            dw = dw32
            if accumulate:
                dw = oracle.accumulate_fp32(out.numpy(), dw32)
            res = torch.from_numpy(np.ascontiguousarray(dw, dtype=np.float32))
        else:
            dwb = oracle.round_bf16_rne(dw32)
            if accumulate:
                dwb = oracle.accumulate_bf16(_bits(out), dwb)
            res = torch.from_numpy(dwb.view(np.int16)).view(torch.bfloat16)
        if out is None:
            return res
        out.copy_(res)  # (copy_ bumps the version counter like the binding does)
        return out

    def zero_pad_rows(self, out, offs, num_groups):
        self.calls.append("zero_pad_rows")
        # the last group end the kernels use: the largest offset clamped to [0, M]
        t = int(np.clip(_offs(offs, num_groups), 0, out.shape[0]).max())
        out[t:] = 0
        return out


def install(monkeypatch) -> StandIns:
    from moe_ragged_bf16_amd import ops
    s = StandIns()
    monkeypatch.setattr(ops, "grouped_det_gemm_fwd", s.fwd)
    monkeypatch.setattr(ops, "grouped_det_gemm_dgrad", s.dgrad)
    monkeypatch.setattr(ops, "grouped_det_gemm_wgrad", s.wgrad)
    monkeypatch.setattr(ops, "zero_pad_rows", s.zero_pad_rows)
    return s
