"""Host check of the decode kernel's aligned-split arithmetic, restated in Python.

The kernel cuts each row's tiles into ranges of equal cost (a sequence with n > 0
tiles costs 4 n + 4 units) and finds the first and last unit holding a split
sequence from its cost prefix alone.  The merge of a split sequence reads one
record from every unit between those two, so the arithmetic must put a piece of
the sequence in each of them.  These cases check that, and that the ranges
partition the tiles, over random batches including empty sequences and far more
units than tiles.  The GPU tests check the kernel's outputs against the oracle.
"""

import numpy as np
import pytest

TILE_COST, PIECE_COST = 4, 4


def split(ctx, units_per_row, floor=True):
    """Per unit: (first tile, end tile, (us, ue) of the sequence its first piece
    continues, or None; (us, ue) of the sequence its last piece runs on with, or None)."""
    n = [(int(c) + 15) // 16 for c in ctx]
    w = [TILE_COST * x + PIECE_COST if x > 0 else 0 for x in n]
    T, W = sum(n), sum(w)
    CC = -(-W // units_per_row)
    if floor:
        CC = max(TILE_COST, CC)
    P = np.concatenate([[0], np.cumsum(w)[:-1]]).astype(int)
    S = np.concatenate([[0], np.cumsum(n)[:-1]]).astype(int)
    cw = np.cumsum(w)

    def at(b):
        if b >= W:
            return T, None
        i = int(np.searchsorted(cw, b, side="right"))
        x = b - P[i] - PIECE_COST
        t = min(0 if x <= 0 else (x + TILE_COST - 1) // TILE_COST, n[i])
        cut = None
        if 0 < t < n[i]:
            cut = ((P[i] + PIECE_COST) // CC, (P[i] + PIECE_COST + TILE_COST * (n[i] - 1)) // CC, i)
        return S[i] + t, cut

    out = []
    for k in range(units_per_row):
        b0 = k * CC
        if b0 >= W:
            out.append((T, T, None, None))
            continue
        t0, first = at(b0)
        t1, last = at(min(b0 + CC, W))
        out.append((t0, t1, first, last))
    return out, n, S


def check(ctx, units_per_row, floor=True):
    units, n, S = split(ctx, units_per_row, floor)
    pos = 0
    for t0, t1, _, _ in units:
        if t1 > t0:
            assert t0 == pos
            pos = t1
    assert pos == sum(n)
    holders = {}
    for k, (t0, t1, _, _) in enumerate(units):
        if t1 <= t0:
            continue  # a unit with no tiles holds no piece
        for i in range(len(n)):
            if n[i] and S[i] < t1 and S[i] + n[i] > t0:
                holders.setdefault(i, []).append(k)
    for i, ks in holders.items():
        if len(ks) == 1:
            continue
        us, ue = ks[0], ks[-1]
        assert ks == list(range(us, ue + 1)), (i, ks)
        for k in ks:
            _, _, first, last = units[k]
            if k > us:
                assert first == (us, ue, i), (i, k, first)
            if k < ue:
                assert last == (us, ue, i), (i, k, last)


@pytest.mark.parametrize("seed", range(6))
def test_split_ranges_partition_tiles_and_holders_are_contiguous(seed):
    rng = np.random.default_rng([70, seed])
    for _ in range(300):
        S = int(rng.integers(1, 40))
        units = int(rng.integers(1, 300))
        kind = int(rng.integers(0, 3))
        if kind == 0:
            ctx = rng.integers(0, 200, S)
        elif kind == 1:
            ctx = rng.integers(0, 3000, S)
        else:
            ctx = np.where(rng.random(S) < 0.3, 0, rng.integers(1, 40, S))
        check(ctx, units)


def test_split_of_the_tiny_workload_with_many_units():
    check([2, 16, 17, 34], 1024)
    check([1, 15, 16, 33], 1)


def test_without_the_one_tile_floor_a_holder_is_skipped():
    """A planted mistake: ranges shorter than one tile's cost leave units without a
    piece between a split sequence's first and last holder."""
    with pytest.raises(AssertionError):
        check([2, 16, 17, 34], 1024, floor=False)
