"""The C-ABI library loads, exports every declared symbol, and refuses bad
arguments before touching the device (no GPU needed).

Pointers below are fake, aligned addresses: every case returns before any
device access, which is what the header promises for validation errors.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import moe_ragged_bf16_amd as mdg
from moe_ragged_bf16_amd import _capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ragged_bf16.h")

OK, EINVAL, EUNSUP, EOVERLAP, EWS, EHIP, ENOMEM = range(7)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = "\n".join(ln for ln in src.splitlines() if not ln.lstrip().startswith("#"))
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return mdg.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(_capi.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_library_exports_exactly_the_declared_symbols(lib):
    """Built with hidden visibility: the dynamic symbol table holds the header's
    entry points and nothing else of the library's own code."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _capi._build.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.split() and ln.split()[1] in "TtWw"}
    ours = {n for n in exported if not n.startswith("_")}   # compiler/runtime glue starts with _
    assert ours == set(declared_functions()), sorted(ours ^ set(declared_functions()))


def test_device_code_has_no_packed_fp32_arithmetic():
    """The library's gfx950 code object, disassembled, holds MFMAs and no packed
    fp32 add, multiply or fma (the build flag that forbids them is effective)."""
    from moe_ragged_bf16_amd import build
    assert build.check_no_packed_fp32(build.LIB_PATH) > 1000


def test_abi_version_and_status_strings(lib):
    assert lib.grouped_det_gemm_abi_version() == 6
    for s in range(7):
        assert mdg.status_string(s)
    assert mdg.status_string(99) == "unknown status"


A, B, C, D, WS = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


@pytest.mark.parametrize("fn", ["grouped_det_gemm_fwd", "grouped_det_gemm_dgrad"])
def test_fwd_dgrad_refusals(lib, fn):
    f = getattr(lib, fn)
    wsf = getattr(lib, fn + "_workspace_bytes")
    need = wsf(8, 256, 256, 4)
    assert need > 0

    def call(a=A, w=B, o=C, d=D, M=8, N=256, K=256, E=4, ws=WS, wsb=None):
        return f(a, w, o, d, M, N, K, E, ws, need if wsb is None else wsb, None)

    # sizes
    assert call(M=-1) == EINVAL
    assert call(N=0) == EINVAL
    assert call(E=0) == EINVAL
    assert call(N=100) == EUNSUP       # n % 8
    assert call(K=100) == EUNSUP       # k % 8
    for n, k in [(96, 256), (256, 72), (8, 8), (264, 1032)]:   # multiples of 8 are sized, not refused
        assert wsf(8, n, k, 4) > 0 and call(N=n, K=k, wsb=0) == EWS
    assert call(E=1025) == EUNSUP      # too many groups
    # pointers
    assert call(a=0) == EINVAL
    assert call(w=0) == EINVAL
    assert call(o=0) == EINVAL
    assert call(d=0) == EINVAL
    assert call(a=A + 8) == EINVAL     # 16-byte alignment
    assert call(o=C + 2) == EINVAL     # offs needs 4 bytes
    # workspace
    assert call(ws=0) == EWS
    assert call(wsb=need - 1) == EWS
    assert call(ws=WS + 16) == EINVAL  # 256-byte alignment
    # overlap of the output with each input and the workspace, of the workspace with the inputs
    assert call(d=A + 16) == EOVERLAP
    assert call(d=B + 4096) == EOVERLAP
    assert call(d=C - 16) == EOVERLAP
    assert call(ws=D) == EOVERLAP
    assert call(ws=A) == EOVERLAP
    assert call(ws=B) == EOVERLAP
    # zero rows: nothing to do, nothing enqueued; row tensors may then be NULL
    need0 = wsf(0, 256, 256, 4)
    assert call(M=0, wsb=need0) == OK
    assert call(a=0, d=0, M=0, wsb=need0) == OK
    assert call(o=0, M=0, wsb=need0) == EINVAL      # offs is always needed


def test_offs_plus_one_is_accepted_alignment(lib):
    # the m_indptr form passes m_indptr + 1: 4-byte aligned only
    need = lib.grouped_det_gemm_fwd_workspace_bytes(0, 256, 256, 4)
    assert lib.grouped_det_gemm_fwd(A, B, C + 4, D, 0, 256, 256, 4, WS, need, None) == OK


@pytest.mark.parametrize("M,N,K,E", [(512, 256, 256, 4), (16384, 14336, 4096, 8), (0, 256, 64, 1),
                                     (65536, 2048, 7168, 256), (100, 512, 64, 1000)])
def test_fwd_dgrad_workspace_rule(lib, M, N, K, E):
    """8 KiB plan head + fp32 256 x 256 partial tiles for min(256, 8 * units) pieces,
    units bounded by (row tiles + one partial tile per group) x column tiles."""
    for fn, cols in (("grouped_det_gemm_fwd_workspace_bytes", N),
                     ("grouped_det_gemm_dgrad_workspace_bytes", K)):
        units = (-(-M // 256) + E) * -(-cols // 256)
        want = 8192 + min(256, 8 * units) * 256 * 256 * 4
        assert getattr(lib, fn)(M, N, K, E) == want, fn
        assert getattr(lib, fn)(M, N + 1, K, E) == 0      # invalid sizes


def test_wgrad_refusals(lib):
    f = lib.grouped_det_gemm_wgrad
    need = lib.grouped_det_gemm_wgrad_workspace_bytes(512, 256, 256, 4)
    assert need > 0
    args = dict(dt=1, acc=0, M=512, N=256, K=256, E=4, ws=WS, wsb=need)

    def call(g=A, x=B, o=C, d=D, **kw):
        a = dict(args)
        a.update(kw)
        return f(g, x, o, d, a["dt"], a["acc"], a["M"], a["N"], a["K"], a["E"], a["ws"], a["wsb"], None)

    assert call(dt=2) == EINVAL                        # bad dtype code
    assert call(dt=0, acc=1, ws=0) == EWS              # bf16 accumulate is offered: checks go on
    assert call(ws=0) == EWS                           # no workspace
    assert call(wsb=need - 1) == EWS                   # short workspace
    assert call(ws=WS + 16) == EINVAL                  # workspace alignment
    assert call(d=A + 64) == EOVERLAP                  # dW over g
    assert call(d=B) == EOVERLAP                       # dW over x
    assert call(d=C - 64) == EOVERLAP                  # dW over offs
    assert call(ws=D + 256) == EOVERLAP                # workspace over dW
    assert call(ws=A) == EOVERLAP                      # workspace over g
    assert call(M=-1) == EINVAL
    assert call(N=300) == EUNSUP
    # accumulate over zero rows leaves dW unchanged: nothing enqueued
    need0 = lib.grouped_det_gemm_wgrad_workspace_bytes(0, 256, 256, 4)
    assert call(M=0, acc=1, wsb=need0) == OK
    assert call(M=0, acc=1, dt=0, wsb=need0) == OK
    assert call(g=0, x=0, M=0, acc=1, wsb=need0) == OK
    assert call(g=0, M=8) == EINVAL
    assert call(d=A + 64, dt=0, acc=1) == EOVERLAP     # bf16 dW over g


def test_zero_pad_rows_refusals(lib):
    f = lib.grouped_det_gemm_zero_pad_rows

    def call(o=C, offs=D, M=8, rb=512, E=4):
        return f(o, offs, M, rb, E, None)

    assert call(M=-1) == EINVAL
    assert call(rb=0) == EINVAL
    assert call(E=0) == EINVAL
    assert call(E=1025) == EUNSUP
    assert call(rb=520) == EUNSUP                      # row bytes % 16
    assert call(rb=(1 << 24) + 16) == EUNSUP
    assert call(offs=0) == EINVAL
    assert call(o=0) == EINVAL
    assert call(o=C + 8) == EINVAL                     # 16-byte alignment
    assert call(offs=D + 2) == EINVAL                  # 4-byte alignment
    assert call(offs=C + 8 * 512 - 4) == EOVERLAP      # offs inside out
    assert call(offs=C - 12) == EOVERLAP               # offs[3] is out's first 4 bytes
    assert call(M=0) == OK                             # nothing to do, nothing enqueued
    assert call(o=0, M=0) == OK


def test_chunk_rows_rule(lib):
    for (M, N, K, E) in [(512, 256, 256, 4), (16384, 14336, 4096, 8), (32768, 1536, 2048, 64),
                         (32768, 4096, 7168, 128), (65536, 2048, 7168, 256), (0, 256, 64, 1),
                         (100000, 256, 64, 1)]:
        r = lib.grouped_det_gemm_wgrad_chunk_rows(M, N, K, E)
        assert r >= 256 and r % 64 == 0
        assert r == lib.grouped_det_gemm_wgrad_chunk_rows(M, N, K, E)
    # big tiles per expert: no split at all for the 8-expert Mixtral-like shape
    assert lib.grouped_det_gemm_wgrad_chunk_rows(16384, 14336, 4096, 8) >= 16384
    assert lib.grouped_det_gemm_wgrad_chunk_rows(8, 204, 64, 1) == 0      # invalid sizes


@pytest.mark.parametrize("M,N,K,E", [(512, 256, 256, 4), (5000, 256, 64, 3), (65536, 2048, 7168, 256),
                                     (32768, 1536, 2048, 64), (1000, 256, 128, 1)])
def test_workspace_covers_every_grouping(lib, M, N, K, E):
    """The workspace bound holds for any split of M rows into E groups."""
    R = lib.grouped_det_gemm_wgrad_chunk_rows(M, N, K, E)
    # partial-tile slots the library provisions: floor(M/R) + #experts with > R rows
    big = min(E, M // (R + 1))
    slots_cap = 0 if big == 0 else M // R + big
    # workspace = 4 KiB head + the fp32 partial tiles (G and X are read in place)
    assert lib.grouped_det_gemm_wgrad_workspace_bytes(M, N, K, E) == \
        -(-(4096 + slots_cap * N * K * 4) // 256) * 256
    have = slots_cap * N * K * 4
    rng = np.random.default_rng(M + E)
    cases = [np.full(E, M // E) for _ in range(1)]
    cases.append(np.array([M] + [0] * (E - 1)))
    for _ in range(200):
        p = rng.dirichlet(np.full(E, rng.choice([0.05, 0.3, 1.0, 5.0])))
        cases.append(rng.multinomial(M, p))
    if E > 1:
        cases.append(np.array([R + 1] * min(E, M // (R + 1)) + [0] * (E - min(E, M // (R + 1)))))
    for s in cases:
        slots = sum(-(-int(m) // R) for m in s if m > R)
        assert slots * N * K * 4 <= have, (s, R)


def _prep(lib, name, *args):
    h = ctypes.c_void_p(0xdead)
    st = getattr(lib, name)(*args, ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("op", ["fwd", "dgrad"])
def test_prepare_fwd_dgrad_refuses_like_one_shot(lib, op):
    one = getattr(lib, "grouped_det_gemm_" + op)
    name = "grouped_det_gemm_prepare_" + op
    need = getattr(lib, "grouped_det_gemm_%s_workspace_bytes" % op)(8, 256, 256, 4)
    bad = [dict(M=-1), dict(N=128), dict(K=100), dict(E=1025), dict(a=0), dict(a=A + 8),
           dict(ws=0), dict(wsb=need - 1), dict(ws=WS + 16), dict(d=A + 16), dict(ws=B)]
    for kw in bad:
        a = dict(a=A, w=B, o=C, d=D, M=8, N=256, K=256, E=4, ws=WS, wsb=need)
        a.update(kw)
        args = (a["a"], a["w"], a["o"], a["d"], a["M"], a["N"], a["K"], a["E"], a["ws"], a["wsb"])
        want = one(*args, None)
        assert want != OK
        st, h = _prep(lib, name, *args)
        assert st == want, kw
        assert h.value is None, kw                     # *launch cleared on error
    assert getattr(lib, name)(A, B, C, D, 8, 256, 256, 4, WS, need, None) == EINVAL


def test_prepare_wgrad_refuses_like_one_shot(lib):
    need = lib.grouped_det_gemm_wgrad_workspace_bytes(512, 256, 256, 4)
    for kw in [dict(dt=2), dict(ws=0), dict(wsb=need - 1), dict(d=A + 64), dict(ws=A), dict(N=300)]:
        a = dict(g=A, x=B, o=C, d=D, dt=1, acc=1, M=512, N=256, K=256, E=4, ws=WS, wsb=need)
        a.update(kw)
        args = (a["g"], a["x"], a["o"], a["d"], a["dt"], a["acc"], a["M"], a["N"], a["K"], a["E"], a["ws"], a["wsb"])
        want = lib.grouped_det_gemm_wgrad(*args, None)
        assert want != OK
        st, h = _prep(lib, "grouped_det_gemm_prepare_wgrad", *args)
        assert st == want and h.value is None, kw


def test_launch_null_and_empty_launches(lib):
    assert lib.grouped_det_gemm_launch(None, None) == EINVAL
    info = _capi.LaunchInfo()
    assert lib.grouped_det_gemm_launch_info(None, ctypes.byref(info)) == EINVAL
    lib.grouped_det_gemm_launch_free(None)             # ignored
    # zero rows: prepared without touching a device; launching enqueues nothing
    need0 = lib.grouped_det_gemm_fwd_workspace_bytes(0, 256, 256, 4)
    st, h = _prep(lib, "grouped_det_gemm_prepare_fwd", 0, B, C, 0, 0, 256, 256, 4, WS, need0)
    assert st == OK and h.value
    assert lib.grouped_det_gemm_launch_info(h, None) == EINVAL
    assert lib.grouped_det_gemm_launch_info(h, ctypes.byref(info)) == OK
    assert (info.op, info.kernels, info.gemm_grid, info.workspace_bytes) == (0, 0, 0, need0)
    assert lib.grouped_det_gemm_launch(h, None) == OK
    lib.grouped_det_gemm_launch_free(h)
    need0 = lib.grouped_det_gemm_wgrad_workspace_bytes(0, 256, 256, 4)
    st, h = _prep(lib, "grouped_det_gemm_prepare_wgrad", 0, 0, C, D, 0, 1, 0, 256, 256, 4, WS, need0)
    assert st == OK
    assert lib.grouped_det_gemm_launch_info(h, ctypes.byref(info)) == OK
    assert (info.op, info.kernels, info.accumulate, info.dw_dtype) == (2, 0, 1, 0)
    assert lib.grouped_det_gemm_launch(h, None) == OK
    lib.grouped_det_gemm_launch_free(h)


def test_missing_library_fails_loudly(monkeypatch):
    """No fallback: without the built library every entry raises."""
    from moe_ragged_bf16_amd import build as _build
    monkeypatch.setattr(_capi, "_lib", None)
    monkeypatch.setattr(_build, "LIB_PATH", "/nonexistent/libmoe_ragged_bf16.so")
    with pytest.raises(ImportError, match="build"):
        mdg.wgrad_workspace_bytes(512, 256, 256, 4)
    with pytest.raises(ImportError):
        mdg.load_library()


def test_fwd_noalloc_refusals_before_the_device(lib):
    """The allocation-free fwd takes fwd's arguments without a workspace and
    refuses the same bad ones before touching the device; no rows: nothing to do."""
    f = lib.grouped_det_gemm_fwd_noalloc

    def call(a=A, w=B, o=C, d=D, M=8, N=256, K=256, E=4):
        return f(a, w, o, d, M, N, K, E, None)

    assert call(M=-1) == EINVAL
    assert call(N=100) == EUNSUP
    assert call(E=1025) == EUNSUP
    assert call(w=0) == EINVAL
    assert call(a=A + 8) == EINVAL
    assert call(o=C + 2) == EINVAL
    assert call(M=0, a=0, d=0) == OK
