"""Split-KV work partition, integer specification (oracle; test infrastructure only).

The pages give the objective, not a scheme: a synchronous attention step ends
with its slowest worker, so the load that matters is the maximum over workers
(Analytical Provisioning, §3.3 "Cycle time": the barrier load is the max of
the per-worker token loads), and attention time grows linearly with the token
load (same paper, §3.1).  The partition below is this library's own integer
rule for making that maximum as small as possible on one GPU: cut the step's
total page work into equal contiguous shares, one per worker.  It is pinned
bit-for-bit against the device planner.

Definitions (all integers):

* A stream is one (request b, KV unit j) pair, j < U, in b-major order; U is
  the number of KV heads for GQA and 1 for MLA.  Stream (b, j) owns
  pages_b = ceil(L_b / P) work units, one per page, in logical page order.
* cp = exclusive prefix sum of pages_b (B + 1 entries); stream (b, j) covers
  units [start, end) with start = U * cp[b] + j * pages_b, end = start + pages_b.
  W = U * cp[B] units in total.
* A = min(G, W) workers are active (G launched); the others have no share.
* Cut points c_g = floor(g * W / A) for g = 0..A; worker g < A processes
  units [c_g, c_{g+1}), never an empty range because W >= A.
* The cursor of unit w < W is (b, j, p) with start(b, j) + p = w; the cursor
  of W is (B, 0, 0).
* A piece is the part of one stream inside one worker's range.  Its result is
  final when the piece is the whole stream; otherwise it is a partial stored in
  slot g when the piece begins at c_g (the worker's first piece) and in slot
  A + g otherwise (then it is the worker's last piece).  2A slots suffice.
* The pieces of a non-empty stream come from the consecutive workers
  first_worker .. first_worker + piece_count - 1 in token order; first_worker
  is the largest g with c_g <= start.  Empty streams (L_b = 0) have
  first_worker = -1 and piece_count = 0.

Here every quantity is found by direct search and enumeration; the device
derives first_worker and piece_count in closed form from (start, end, W, A),
which the GPU tests compare with these values.
"""
from __future__ import annotations

import dataclasses
from typing import List, Tuple

import numpy as np


@dataclasses.dataclass
class Partition:
    cp: np.ndarray            # int64 [B+1]
    total: int                # W
    active: int               # A = min(G, W)
    cuts: np.ndarray          # int64 [A+1]
    cursors: np.ndarray       # int64 [A+1][3] (b, j, p) of unit cuts[g]
    first_worker: np.ndarray  # int64 [B*U]
    piece_count: np.ndarray   # int64 [B*U]
    pieces: List[Tuple[int, int, int, int, int, int]]   # (g, b, j, p0, p1, slot)


def _stream_of(w: int, cp: np.ndarray, U: int, B: int):
    """(b, j, p) of unit w < W, by direct search (largest b with U*cp[b] <= w)."""
    b = int(np.searchsorted(U * cp, w, side="right")) - 1
    pages = int(cp[b + 1] - cp[b])
    off = w - U * int(cp[b])
    return b, off // pages, off % pages


def partition(seq_lens, page_size: int, units: int, workers: int) -> Partition:
    L = np.asarray(seq_lens, dtype=np.int64)
    B = len(L)
    U = int(units)
    G = int(workers)
    pages = (L + page_size - 1) // page_size
    cp = np.zeros(B + 1, dtype=np.int64)
    cp[1:] = np.cumsum(pages)
    W = U * int(cp[B])
    A = min(G, W)

    cuts = np.array([(g * W) // A for g in range(A + 1)] if A else [0], dtype=np.int64)

    cursors = np.zeros((A + 1, 3), dtype=np.int64)
    for g in range(A + 1):
        c = int(cuts[g])
        cursors[g] = (B, 0, 0) if c >= W else _stream_of(c, cp, U, B)

    pieces = []
    for g in range(A):
        lo, hi = int(cuts[g]), int(cuts[g + 1])
        w = lo
        while w < hi:
            b, j, p = _stream_of(w, cp, U, B)
            start = U * int(cp[b]) + j * int(pages[b])
            end = start + int(pages[b])
            stop = min(end, hi)
            p0, p1 = w - start, stop - start
            if p0 == 0 and p1 == pages[b]:
                slot = -1
            elif w == lo:
                slot = g
            else:
                slot = A + g
            pieces.append((g, b, j, p0, p1, slot))
            w = stop

    first_worker = np.full(B * U, -1, dtype=np.int64)
    piece_count = np.zeros(B * U, dtype=np.int64)
    for g, b, j, p0, p1, slot in pieces:
        s = b * U + j
        if first_worker[s] < 0:
            first_worker[s] = g
        piece_count[s] += 1
    return Partition(cp, W, A, cuts, cursors, first_worker, piece_count, pieces)
