"""ctypes loader of the gfx950 HIP library (``libmoe_ragged_bf16.so``).

Argument marshalling only.  The library is required: if it is missing or fails
to load, every call raises; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

from . import build as _build

MDG_OK, MDG_EINVAL, MDG_EUNSUPPORTED, MDG_EOVERLAP, MDG_EWORKSPACE, MDG_EHIP, MDG_ENOMEM = range(7)
MDG_BF16, MDG_FP32 = 0, 1

EXPORTED = (
    "grouped_det_gemm_abi_version",
    "grouped_det_gemm_status_string",
    "grouped_det_gemm_fwd",
    "grouped_det_gemm_dgrad",
    "grouped_det_gemm_fwd_noalloc",
    "grouped_det_gemm_fwd_workspace_bytes",
    "grouped_det_gemm_dgrad_workspace_bytes",
    "grouped_det_gemm_wgrad",
    "grouped_det_gemm_wgrad_workspace_bytes",
    "grouped_det_gemm_wgrad_chunk_rows",
    "grouped_det_gemm_zero_pad_rows",
    "grouped_det_gemm_prepare_fwd",
    "grouped_det_gemm_prepare_dgrad",
    "grouped_det_gemm_prepare_wgrad",
    "grouped_det_gemm_launch",
    "grouped_det_gemm_launch_info",
    "grouped_det_gemm_launch_free",
)


class LaunchInfo(ctypes.Structure):
    """mdg_launch_info of the C header."""
    _fields_ = [("op", ctypes.c_int32), ("device", ctypes.c_int32), ("kernels", ctypes.c_int32),
                ("gemm_grid", ctypes.c_int32), ("dw_dtype", ctypes.c_int32), ("accumulate", ctypes.c_int32),
                ("chunk_rows", ctypes.c_int32), ("tail_slots", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64)]

_lock = threading.Lock()
_lib = None


class MdgError(RuntimeError):
    """A non-OK status returned by the C ABI."""

    def __init__(self, entry: str, status: int, message: str):
        super().__init__(f"{entry}: status {status}: {message}")
        self.entry = entry
        self.status = status


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load (once) and return the library, with argument types declared.  It is
    required: a missing or unloadable library raises (no fallback exists)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = path or _build.LIB_PATH
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build the HIP library first "
                "(python -m moe_ragged_bf16_amd.build)")
        lib = ctypes.CDLL(path)
        i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        lib.grouped_det_gemm_abi_version.restype = ctypes.c_int
        lib.grouped_det_gemm_abi_version.argtypes = []
        lib.grouped_det_gemm_status_string.restype = ctypes.c_char_p
        lib.grouped_det_gemm_status_string.argtypes = [ctypes.c_int]
        for name in ("grouped_det_gemm_fwd", "grouped_det_gemm_dgrad"):
            f = getattr(lib, name)
            f.restype = ctypes.c_int
            f.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp]
        lib.grouped_det_gemm_fwd_noalloc.restype = ctypes.c_int
        lib.grouped_det_gemm_fwd_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp]
        for name in ("grouped_det_gemm_fwd_workspace_bytes", "grouped_det_gemm_dgrad_workspace_bytes"):
            f = getattr(lib, name)
            f.restype = sz
            f.argtypes = [i64, i64, i64, i32]
        lib.grouped_det_gemm_wgrad.restype = ctypes.c_int
        lib.grouped_det_gemm_wgrad.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                                               i64, i64, i64, i32, vp, sz, vp]
        lib.grouped_det_gemm_wgrad_workspace_bytes.restype = sz
        lib.grouped_det_gemm_wgrad_workspace_bytes.argtypes = [i64, i64, i64, i32]
        lib.grouped_det_gemm_wgrad_chunk_rows.restype = i64
        lib.grouped_det_gemm_wgrad_chunk_rows.argtypes = [i64, i64, i64, i32]
        lib.grouped_det_gemm_zero_pad_rows.restype = ctypes.c_int
        lib.grouped_det_gemm_zero_pad_rows.argtypes = [vp, vp, i64, i64, i32, vp]
        pp = ctypes.POINTER(vp)
        for name in ("grouped_det_gemm_prepare_fwd", "grouped_det_gemm_prepare_dgrad"):
            f = getattr(lib, name)
            f.restype = ctypes.c_int
            f.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, pp]
        lib.grouped_det_gemm_prepare_wgrad.restype = ctypes.c_int
        lib.grouped_det_gemm_prepare_wgrad.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                                                       i64, i64, i64, i32, vp, sz, pp]
        lib.grouped_det_gemm_launch.restype = ctypes.c_int
        lib.grouped_det_gemm_launch.argtypes = [vp, vp]
        lib.grouped_det_gemm_launch_info.restype = ctypes.c_int
        lib.grouped_det_gemm_launch_info.argtypes = [vp, ctypes.POINTER(LaunchInfo)]
        lib.grouped_det_gemm_launch_free.restype = None
        lib.grouped_det_gemm_launch_free.argtypes = [vp]
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().grouped_det_gemm_status_string(status).decode()


def check(entry: str, status: int) -> None:
    if status != MDG_OK:
        raise MdgError(entry, status, status_string(status))
