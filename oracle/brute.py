"""Exhaustive enumeration of valid level-order k-d trees for tiny N.

TEST INFRASTRUCTURE (only tests/ may import it). Independent of both the C++
oracle and the HIP library: it tries every arrangement of the N points over
the N level-order slots and keeps those that satisfy the two conditions of
I. Wald, "GPU-friendly, Parallel, and (Almost-)In-Place Construction of
Left-Balanced k-d Trees" (problem statement): every point in a node's left
subtree is <= the node and every point in its right subtree is >= the node,
in the node's split dimension (level mod k); the balancing condition holds by
construction since slots 0..N-1 of a level-order array are the complete
left-balanced shape. Parent of slot i is (i-1)//2 (indexing paragraph).
"""
from __future__ import annotations

import itertools

import numpy as np


def _ancestor_pairs(n: int):
    """(node, ancestor, node_is_in_left_subtree, ancestor_level) for all pairs."""
    out = []
    for node in range(1, n):
        child = node
        while child > 0:
            anc = (child - 1) // 2
            lvl = (anc + 1).bit_length() - 1
            out.append((node, anc, child == 2 * anc + 1, lvl))
            child = anc
    return out


def valid_trees(points, strict: bool = False) -> list[tuple[int, ...]]:
    """All permutations perm (slot -> original index) satisfying the k-d
    condition with float <=/>=; with strict=True, the order is (coordinate,
    original index) with strict inequalities instead."""
    pts = np.asarray(points, dtype=np.float32)
    n, k = pts.shape
    if n > 8:
        raise ValueError("brute force is for N <= 8")
    if n == 0:
        return [()]
    perms = np.array(list(itertools.permutations(range(n))), dtype=np.int64)
    ok = np.ones(len(perms), dtype=bool)
    for node, anc, left, lvl in _ancestor_pairs(n):
        d = lvl % k
        pn = perms[:, node]
        pa = perms[:, anc]
        xn = pts[pn, d]
        xa = pts[pa, d]
        if strict:
            less = (xn < xa) | ((xn == xa) & (pn < pa))
            greater = (xn > xa) | ((xn == xa) & (pn > pa))
            ok &= less if left else greater
        else:
            ok &= (xn <= xa) if left else (xn >= xa)
    return [tuple(int(v) for v in row) for row in perms[ok]]
