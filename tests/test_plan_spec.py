"""Properties of the integer split-KV partition (the oracle's statement of it).

The device planner is compared with it bit-for-bit in the GPU tests; here the
rule itself is checked against what it promises: an exact tiling of every
stream, equal shares (up to one unit), unique partial slots, no empty worker,
and the first-worker / piece-count rule the in-kernel merge relies on.
"""
import numpy as np
import pytest

from oracle.plan import partition


def _check(seq_lens, P, U, G):
    part = partition(seq_lens, P, U, G)
    L = np.asarray(seq_lens, dtype=np.int64)
    pages = (L + P - 1) // P
    B = len(L)
    A = part.active
    assert part.total == U * int(pages.sum())
    assert A == min(G, part.total)
    cuts = part.cuts
    assert len(cuts) == A + 1
    assert cuts[0] == 0 and cuts[-1] == part.total
    if A:
        sizes = np.diff(cuts)
        assert sizes.min() >= 1 and sizes.max() - sizes.min() <= 1
    # every stream tiled exactly, in order, by its pieces from consecutive workers
    by_stream = {}
    for g, b, j, p0, p1, slot in part.pieces:
        assert cuts[g] <= U * part.cp[b] + j * pages[b] + p0 < cuts[g + 1]
        assert p1 > p0
        by_stream.setdefault((b, j), []).append((p0, p1, g, slot))
    for b in range(B):
        for j in range(U):
            s = b * U + j
            ps = by_stream.get((b, j), [])
            if pages[b] == 0:
                assert ps == [] and part.first_worker[s] == -1 and part.piece_count[s] == 0
                continue
            ps.sort()
            assert ps[0][0] == 0 and ps[-1][1] == pages[b]
            for a, c in zip(ps[:-1], ps[1:]):
                assert a[1] == c[0]
            gs = [g for _, _, g, _ in ps]
            assert gs == list(range(gs[0], gs[0] + len(gs)))
            start = U * part.cp[b] + j * pages[b]
            # first worker = largest g with c_g <= start
            assert gs[0] == part.first_worker[s] == int(np.searchsorted(cuts, start, side="right")) - 1
            assert part.piece_count[s] == len(ps)
            if len(ps) == 1:
                assert ps[0][3] == -1
            else:
                assert all(sl >= 0 for *_, sl in ps)
    slots = [s for *_, s in part.pieces if s >= 0]
    assert len(slots) == len(set(slots)) and all(0 <= s < 2 * A for s in slots)
    # cursors name the unit each cut starts at
    for g in range(A + 1):
        c = int(cuts[g])
        b, j, p = part.cursors[g]
        if c == part.total:
            assert (b, j, p) == (B, 0, 0)
        else:
            assert U * part.cp[b] + j * pages[b] + p == c and p < pages[b]
    return part


@pytest.mark.parametrize("seed", range(16))
def test_random_partitions(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    lens = rng.integers(0, 300, size=B)
    lens[rng.random(B) < 0.2] = 0
    P = int(rng.choice([1, 4, 16, 64]))
    U = int(rng.choice([1, 2, 8]))
    G = int(rng.integers(1, 200))
    _check(lens, P, U, G)


def test_more_workers_than_units():
    part = _check([3, 0, 5], 4, 2, 50)
    assert part.active == part.total == 6
    assert all(p[4] - p[3] == 1 for p in part.pieces)


def test_all_empty():
    part = _check([0, 0], 16, 8, 7)
    assert part.total == 0 and part.active == 0 and part.pieces == []
    assert list(part.cuts) == [0]


def test_single_worker_takes_everything_whole():
    part = _check([17, 40, 1], 16, 2, 1)
    assert all(s == -1 for *_, s in part.pieces)


def test_hand_worked_example():
    # lengths 5, 9, 0 tokens, page 4 -> pages 2, 3, 0; one KV unit; 2 workers; W = 5
    part = partition([5, 9, 0], 4, 1, 2)
    assert list(part.cp) == [0, 2, 5, 5] and part.total == 5 and part.active == 2
    assert list(part.cuts) == [0, 2, 5]
    assert part.pieces == [(0, 0, 0, 0, 2, -1), (1, 1, 0, 0, 3, -1)]
    # three workers: cuts 0, 1, 3, 5
    part = partition([5, 9, 0], 4, 1, 3)
    assert list(part.cuts) == [0, 1, 3, 5]
    assert part.pieces == [(0, 0, 0, 0, 1, 0), (1, 0, 0, 1, 2, 1), (1, 1, 0, 0, 1, 4), (2, 1, 0, 1, 3, 2)]
    assert list(part.first_worker) == [0, 1, -1]
    assert list(part.piece_count) == [2, 2, 0]
    # eight workers but only five units: five active workers, one page each
    part = partition([5, 9, 0], 4, 1, 8)
    assert part.active == 5 and list(part.cuts) == [0, 1, 2, 3, 4, 5]
    assert list(part.piece_count) == [2, 3, 0]


def test_balance_under_skew():
    """Equal shares whatever the skew: one 64k-token request among short ones."""
    lens = np.array([65536] + [100] * 255)
    part = _check(lens, 16, 8, 2048)
    sizes = np.diff(part.cuts)
    assert sizes.max() - sizes.min() <= 1
