"""Checker for the split-widest-dimension tree (perm, dims).

TEST INFRASTRUCTURE (see the package docstring).

Source: I. Wald, "GPU-friendly, Parallel, and (Almost-)In-Place Construction
of Left-Balanced k-d Trees" (arXiv 2211.00120), section on the
split-widest-dimension variant. That section also computes a node's domain
without any top-down state: start from the bounding box of all points and
walk from the node up to the root, clipping the box by each ancestor's plane
on the side the node lies. This checker uses that formulation, not the
oracle's top-down recursion:

* every node's split dimension is the widest (float32 extent, lowest
  dimension on ties) of its domain clipped bottom-up, with '<'/'>'
  comparisons as the oracle's reading;
* every node's point is on the correct side of every ancestor's plane, by
  (coordinate in the ancestor's dimension, original index), strictly;
* perm is a permutation of 0 .. N-1 (the shape is fixed by N).

Vectorised over all nodes of a level at once (numpy); returns None when the
tree passes, else a message naming the first failure.
"""
from __future__ import annotations

import numpy as np


def _widest(lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore", over="ignore"):  # inf - inf is NaN, as in C
        ext = (hi - lo).astype(np.float32)
    best = np.zeros(len(ext), dtype=np.int64)
    best_ext = ext[:, 0].copy()
    for d in range(1, ext.shape[1]):
        better = ext[:, d] > best_ext
        best[better] = d
        best_ext[better] = ext[better, d]
    return best


def check(points, perm, dims) -> str | None:
    pts = np.ascontiguousarray(points, dtype=np.float32)
    n, k = pts.shape
    perm = np.asarray(perm, dtype=np.int64)
    dims = np.asarray(dims, dtype=np.int64)
    if perm.shape != (n,) or dims.shape != (n,):
        return "perm and dims must have N entries"
    if n == 0:
        return None
    if not np.array_equal(np.sort(perm), np.arange(n)):
        return "perm is not a permutation"
    if dims.min() < 0 or dims.max() >= k:
        return "dimension out of range"
    box_lo, box_hi = pts.min(0), pts.max(0)
    nodes = np.arange(n)
    x = pts[perm]                      # point of every node
    lo = np.tile(box_lo, (n, 1))
    hi = np.tile(box_hi, (n, 1))
    cur = nodes.copy()                 # the node whose parent is examined next
    alive = cur > 0
    while alive.any():
        c = cur[alive]
        a = (c - 1) // 2               # the ancestor
        s = nodes[alive]               # the node being checked
        d = dims[a]
        plane = x[a, d]
        left = c == 2 * a + 1
        # the node's point against the ancestor's: (coordinate, index) order
        mine, idx = x[s, d], perm[s]
        before = (mine < plane) | ((mine == plane) & (idx < perm[a]))
        after = (mine > plane) | ((mine == plane) & (idx > perm[a]))
        bad = np.flatnonzero(np.where(left, ~before, ~after))
        if len(bad):
            return "node %d is on the wrong side of ancestor %d" % (s[bad[0]], a[bad[0]])
        # clip the node's domain by the ancestor's plane
        rows = s
        hi_d = hi[rows, d]
        lo_d = lo[rows, d]
        hi[rows[left], d[left]] = np.minimum(hi_d[left], plane[left])
        lo[rows[~left], d[~left]] = np.maximum(lo_d[~left], plane[~left])
        cur[alive] = a
        alive = cur > 0
    want = _widest(lo, hi)
    bad = np.flatnonzero(want != dims)
    if len(bad):
        s = bad[0]
        return "node %d splits dimension %d, its domain's widest is %d" % (s, dims[s], want[s])
    return None
