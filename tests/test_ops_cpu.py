"""Host-side checks of the one-shot binding that must run before the library is
called (no GPU needed): a caller's workspace is refused unless it is a
contiguous uint8 device tensor of at least the queried size, for fwd, dgrad and
wgrad alike."""
import pytest
import torch

from moe_ragged_bf16_amd import ops


class _NoCalls:
    """Stand-in library: answers the workspace queries, fails on any other call."""

    def __getattr__(self, name):
        if name.endswith("_workspace_bytes"):
            return lambda *a: 4096
        raise AssertionError(f"library entry {name} reached despite a bad workspace")


@pytest.fixture
def host_only(monkeypatch):
    # let CPU tensors through the tensor checks so the workspace check is what refuses
    monkeypatch.setattr(ops, "_need", lambda *a, **k: None)
    monkeypatch.setattr(ops, "_offs_ptr", lambda offs, E: 0)
    monkeypatch.setattr(ops._capi, "load_library", lambda: _NoCalls())


def _args():
    M, N, K, E = 8, 256, 64, 2
    return (torch.zeros((M, K), dtype=torch.bfloat16), torch.zeros((E, N, K), dtype=torch.bfloat16),
            torch.zeros((M, N), dtype=torch.bfloat16), torch.tensor([4, 8], dtype=torch.int32))


BAD = [
    (lambda: torch.empty(8192, dtype=torch.uint8), "ROCm device"),              # host memory
    (lambda: torch.empty(2048, dtype=torch.float32), "contiguous uint8"),       # wrong dtype
    (lambda: torch.empty(1, dtype=torch.uint8).expand(8192), "contiguous uint8"),  # stride-0 view
    (lambda: torch.empty((64, 256), dtype=torch.uint8)[:, ::2], "contiguous uint8"),  # strided view
    (lambda: "not a tensor", "contiguous uint8"),
]


@pytest.mark.parametrize("make,msg", BAD)
@pytest.mark.parametrize("op", ["fwd", "dgrad", "wgrad"])
def test_bad_workspace_refused_before_the_library_call(host_only, op, make, msg):
    x, w, g, offs = _args()
    ws = make()
    with pytest.raises(ValueError, match=msg):
        if op == "fwd":
            ops.grouped_det_gemm_fwd(x, w, offs, workspace=ws)
        elif op == "dgrad":
            ops.grouped_det_gemm_dgrad(g, w, offs, workspace=ws)
        else:
            ops.grouped_det_gemm_wgrad(g, x, offs, out_dtype=torch.float32, workspace=ws)


@pytest.mark.parametrize("op", ["fwd", "dgrad", "wgrad"])
def test_small_workspace_refused(host_only, op):
    x, w, g, offs = _args()
    ws = torch.empty(4095, dtype=torch.uint8)     # the stand-in library asks for 4096
    with pytest.raises(ValueError, match="too small"):
        if op == "fwd":
            ops.grouped_det_gemm_fwd(x, w, offs, workspace=ws)
        elif op == "dgrad":
            ops.grouped_det_gemm_dgrad(g, w, offs, workspace=ws)
        else:
            ops.grouped_det_gemm_wgrad(g, x, offs, out_dtype=torch.float32, workspace=ws)
