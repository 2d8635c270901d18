"""The fwd/dgrad work plan restated for tests: how many 256 x 256 units a call
has and which of them the tail split cuts (so tests can assert which cases
exercise a split).  Mirrors the rule the C ABI header documents: with U units,
T = U mod 256 tail units are cut into S = min(256 // T, 8, groups of 4
reduction stages, slots // T) pieces when S >= 2."""
import math

BALANCE, MAX_SPLIT = 256, 8


def units(op, sizes, N, K):
    n_j = math.ceil(N / 256) if op == "fwd" else math.ceil(K / 256)
    return sum(math.ceil(int(m) / 256) for m in sizes) * n_j


def slots(op, M, N, K, E):
    n_j = math.ceil(N / 256) if op == "fwd" else math.ceil(K / 256)
    return min(BALANCE, MAX_SPLIT * (math.ceil(M / 256) + E) * n_j)


def tail_plan(op, sizes, N, K, M=None, E=None):
    """(U, T, S): T split units of S pieces each, (U, 0, 1) when nothing is split."""
    M = int(sum(int(m) for m in sizes)) if M is None else M
    E = len(sizes) if E is None else E
    U = units(op, sizes, N, K)
    T = U % BALANCE
    if T == 0:
        return U, 0, 1
    red = K if op == "fwd" else N
    groups = ((red + 31) // 32 + 3) // 4
    S = min(BALANCE // T, MAX_SPLIT, groups, slots(op, M, N, K, E) // T)
    return (U, T, S) if S >= 2 else (U, 0, 1)


def unit_tiles(op, sizes, N, K):
    """(group, row tile, column tile) of every unit in unit order: groups in
    order; within a group, panels of 4 row tiles walked column by column (the
    order the device scheduler numbers a group's units in)."""
    n_j = math.ceil(N / 256) if op == "fwd" else math.ceil(K / 256)
    out = []
    for e, m in enumerate(sizes):
        rows = math.ceil(int(m) / 256)
        for ul in range(rows * n_j):
            per_panel = 4 * n_j
            panel = ul // per_panel
            r0 = panel * 4
            h = min(4, rows - r0)
            rem = ul - panel * per_panel
            out.append((e, r0 + rem % h, rem // h))
    return out


def split_mask(op, sizes, N, K, M=None, E=None):
    """Boolean [sum(sizes), n_j] array: True where a (row, column tile) belongs to
    a unit the tail split cuts, plus the plan (U, T, S)."""
    import numpy as np
    U, T, S = tail_plan(op, sizes, N, K, M, E)
    n_j = math.ceil(N / 256) if op == "fwd" else math.ceil(K / 256)
    starts = np.concatenate([[0], np.cumsum(np.asarray(sizes, dtype=np.int64))])
    mask = np.zeros((int(starts[-1]), n_j), dtype=bool)
    if T:
        for e, rt, ct in unit_tiles(op, sizes, N, K)[U - T:]:
            r0 = int(starts[e]) + 256 * rt
            r1 = min(int(starts[e + 1]), r0 + 256)
            mask[r0:r1, ct] = True
    return mask, (U, T, S)
