"""The tail-split cases of tests/test_gpu_tail_split.py exercise what they claim."""
from _plan import tail_plan
from test_gpu_tail_split import CASES


def test_cases_cover_the_plan_shapes():
    seen = {}
    for sizes, N, K, pad, want in CASES:
        for op in ("fwd", "dgrad"):
            U, T, S = tail_plan(op, sizes, N, K, M=sum(sizes) + pad)
            seen.setdefault(S, []).append((op, sizes, N, K))
            if op in want:
                assert S == want[op], (op, sizes, N, K, U, T, S)
    assert 8 in seen and 1 in seen and any(2 <= s < 8 for s in seen), seen


def test_plan_rule_examples():
    # Mixtral-like dgrad: 67 row tiles x 16 column tiles = 1072 units, 48 left after 4 rounds
    sizes = [2048] * 8
    assert tail_plan("fwd", sizes, 14336, 4096) == (64 * 56, 0, 1)       # whole rounds: no split
    U, T, S = tail_plan("dgrad", [2100, 2000, 2048, 2048, 1990, 2100, 2050, 2048], 14336, 4096)
    assert (T, S) == (U % 256, 256 // T if 256 // T <= 8 else 8)
    assert tail_plan("fwd", [4352], 2048, 256) == (136, 0, 1)            # T = 136 > 128: no split
