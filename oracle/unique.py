"""Duplicate-removal oracle.

TEST INFRASTRUCTURE (see the package docstring).

Source: J. Robinson, "An Implementation of a Balanced Kd Tree Builder Using
GPUs" (KdTreeGPU wiki), the duplicate-removal section: with the tuples
sorted by all their coordinates (the primary one first, then the next, and
so on), tuples that are equal in every coordinate are adjacent, and all but
one of each such run are removed. The page also states that two tuples are
equal only if all their coordinates are equal.

Readings fixed here: coordinates compare with IEEE '==' (so -0.0 equals
+0.0; NaN is outside the definition); of each group of equal tuples the one
kept is the one with the smallest original index; the output lists the kept
indices in increasing order, so it does not depend on the sort.
"""
from __future__ import annotations

import numpy as np


def unique_indices(points) -> np.ndarray:
    """Ascending original indices of one representative (the smallest index)
    of every distinct tuple."""
    pts = np.ascontiguousarray(points, dtype=np.float32)
    n = pts.shape[0]
    if n == 0:
        return np.zeros(0, dtype=np.int32)
    canon = pts + np.float32(0.0)  # -0.0 + 0.0 = +0.0: one spelling of zero
    order = np.lexsort(tuple(canon[:, d] for d in reversed(range(pts.shape[1]))) + ())
    # stable lexsort keeps index order inside each run of equal tuples
    s = canon[order]
    head = np.ones(n, dtype=bool)
    head[1:] = (s[1:] != s[:-1]).any(axis=1)
    return np.sort(order[head]).astype(np.int32)
