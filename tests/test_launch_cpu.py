"""Host-side refusals of the prepared-launch functions (no GPU needed: every
case is refused before the library is asked to bind anything)."""
import pytest
import torch

import moe_ragged_bf16_amd as mdg


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def test_prepare_refuses_host_tensors_and_bad_arguments():
    x, w, g = _t(8, 64), _t(2, 256, 64), _t(8, 256)
    offs = torch.tensor([4, 8], dtype=torch.int32)
    with pytest.raises(ValueError, match="ROCm device"):
        mdg.prepare_grouped_det_gemm_fwd(x, w, offs)
    with pytest.raises(ValueError, match="ROCm device"):
        mdg.prepare_grouped_det_gemm_dgrad(g, w, offs)
    with pytest.raises(TypeError, match="bool"):
        mdg.prepare_grouped_det_gemm_wgrad(g, x, offs, accumulate=1)
    with pytest.raises(TypeError, match="bfloat16"):
        mdg.prepare_grouped_det_gemm_fwd(x.float(), w, offs)


def test_accumulate_modes_and_names():
    assert mdg.ACCUMULATE_MODES == ("off", "fused")
    for name in ("prepare_grouped_det_gemm_fwd", "prepare_grouped_det_gemm_dgrad",
                 "prepare_grouped_det_gemm_wgrad", "GroupedDetGemmLaunch"):
        assert hasattr(mdg, name)
