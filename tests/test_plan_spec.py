"""Properties of the integer split-KV partition (the oracle's statement of it).

The device planner is compared with it bit-for-bit in the GPU tests; here the
rule itself is checked against what it promises: an exact tiling of every
stream, equal shares (up to one unit, before snapping), unique partial slots,
and the first-worker rule the merge relies on.
"""
import numpy as np
import pytest

from oracle.plan import partition


def _check(seq_lens, P, U, G, snap):
    part = partition(seq_lens, P, U, G, snap)
    L = np.asarray(seq_lens, dtype=np.int64)
    pages = (L + P - 1) // P
    B = len(L)
    assert part.total == U * int(pages.sum())
    cuts = part.cuts
    assert cuts[0] == 0 and cuts[-1] == part.total and np.all(np.diff(cuts) >= 0)
    if snap == 0:
        sizes = np.diff(cuts)
        if G:
            assert sizes.max() - sizes.min() <= 1
    # every stream tiled exactly, in order, by its pieces
    by_stream = {}
    for g, b, j, p0, p1, slot in part.pieces:
        assert cuts[g] <= U * part.cp[b] + j * pages[b] + p0 < cuts[g + 1] or p0 == p1
        assert p1 > p0
        by_stream.setdefault((b, j), []).append((p0, p1, g, slot))
    for b in range(B):
        for j in range(U):
            ps = by_stream.get((b, j), [])
            if pages[b] == 0:
                assert ps == [] and part.first_worker[b * U + j] == -1
                continue
            ps.sort()
            assert ps[0][0] == 0 and ps[-1][1] == pages[b]
            for a, c in zip(ps[:-1], ps[1:]):
                assert a[1] == c[0]
            assert ps[0][2] == part.first_worker[b * U + j]
            if len(ps) == 1:
                assert ps[0][3] == -1
            else:
                assert all(s >= 0 for *_, s in ps)
                assert [g for _, _, g, _ in ps] == sorted(g for _, _, g, _ in ps)
    slots = [s for *_, s in part.pieces if s >= 0]
    assert len(slots) == len(set(slots)) and all(0 <= s < 2 * G for s in slots)
    # cursors name the unit each cut starts at
    for g in range(G + 1):
        c = int(cuts[g])
        b, j, p = part.cursors[g]
        if c == part.total:
            assert (b, j, p) == (B, 0, 0)
        else:
            assert U * part.cp[b] + j * pages[b] + p == c and p < pages[b]
    return part


@pytest.mark.parametrize("seed", range(12))
def test_random_partitions(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    lens = rng.integers(0, 300, size=B)
    lens[rng.random(B) < 0.2] = 0
    P = int(rng.choice([1, 4, 16, 64]))
    U = int(rng.choice([1, 2, 8]))
    G = int(rng.integers(1, 200))
    snap = int(rng.choice([0, 0, 1, 3, 10]))
    _check(lens, P, U, G, snap)


def test_more_workers_than_units():
    part = _check([3, 0, 5], 4, 2, 50, 0)
    assert sum(1 for g in range(50) if part.cuts[g + 1] > part.cuts[g]) == part.total


def test_all_empty():
    part = _check([0, 0], 16, 8, 7, 0)
    assert part.total == 0 and part.pieces == []


def test_single_worker_takes_everything_whole():
    part = _check([17, 40, 1], 16, 2, 1, 0)
    assert all(s == -1 for *_, s in part.pieces)


def test_snapping_avoids_short_pieces():
    lens = [64 * 52, 64 * 3, 64 * 47]          # W = 102 pages; the raw cut at 51 leaves 1 page
    part0 = partition(lens, 64, 1, 2, 0)
    part = _check(lens, 64, 1, 2, 8)
    assert list(part.cuts) == [0, 52, 102]
    short0 = [p for p in part0.pieces if p[4] - p[3] < 8 and p[5] >= 0]
    short = [p for p in part.pieces if p[4] - p[3] < 8 and p[5] >= 0]
    assert short0 and not short


def test_hand_worked_example():
    # lengths 5, 9, 0 tokens, page 4 -> pages 2, 3, 0; one KV unit; 2 workers; W = 5
    part = partition([5, 9, 0], 4, 1, 2, 0)
    assert list(part.cp) == [0, 2, 5, 5] and part.total == 5
    assert list(part.cuts) == [0, 2, 5]
    assert part.pieces == [(0, 0, 0, 0, 2, -1), (1, 1, 0, 0, 3, -1)]
    # three workers: cuts 0, 1, 3, 5
    part = partition([5, 9, 0], 4, 1, 3, 0)
    assert list(part.cuts) == [0, 1, 3, 5]
    assert part.pieces == [(0, 0, 0, 0, 1, 0), (1, 0, 0, 1, 2, 1), (1, 1, 0, 0, 1, 4), (2, 1, 0, 1, 3, 2)]
    assert list(part.first_worker) == [0, 1, -1]
