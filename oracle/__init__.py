"""CPU oracle for the deterministic ragged BF16 grouped GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the HIP
library and its Python binding) never imports, links or calls it, and shares no
code with it: this package is plain NumPy, written from the definitions on the
pages, and is pinned in the CPU tests by brute force, closed forms and
invariants.

Sources it follows:

* "Cake ragged BF16 grouped GEMM (experimental)" API page (docs.flashinfer.ai),
  introduction and operations table: groups are consecutive row ranges given by
  ``offs[E]`` (cumulative end offsets) or ``m_indptr[E + 1]``; fwd
  ``Y[g] = X[g] @ W[e].T``, dgrad ``dX[g] = G[g] @ W[e]``, wgrad
  ``dW[e] = G[g].T @ X[g]``; bf16 operands; empty groups give exactly-zero weight
  gradients.
* flashinfer PR #8924 ("det-only names ... deterministic weight-gradient
  accumulation"), section "Design and numerics": an accumulate into an fp32 out
  gives ``RN32(out + dW)``; the bf16 dW is added in bf16 for a bf16 out; and its
  "Tests" description, which checks the GPU programs against an fp64 reference.

Every function here is pinned (no function is "parity unpinned"); the pins are
listed in ``tests/test_oracle_pins.py``.
"""
from .grouped_gemm import (  # noqa: F401
    widen_bf16,
    round_bf16_rne,
    group_ranges,
    offs_from_indptr,
    fwd,
    dgrad,
    wgrad,
    fwd_rows,
    dgrad_rows,
    wgrad_expert,
    accumulate_fp32,
    accumulate_bf16,
)
