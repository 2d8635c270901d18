"""The C ABI from a C++ caller with no Python in between (tests/c_abi_smoke.cpp:
workspace queries, refusals, a prepared fwd launched twice, one-shot dgrad,
wgrad and both fused accumulates, each against a closed form)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_smoke")


def test_c_abi_smoke_program():
    assert os.path.exists(BIN), "tests/c_abi_smoke is missing: run __graft_entry__.build()"
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c abi smoke ok" in res.stdout
