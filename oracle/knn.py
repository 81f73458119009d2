"""Brute-force k-nearest-neighbour oracle.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.

Source: F. Gieseke et al., "Bigger Buffer k-d Trees on Multi-Many-Core
Systems" (arXiv 1512.02831), section 2.3 ("Nearest Neighbor Search via K-d
Trees") and the problem statement before it: the K nearest neighbours of
every query point among the reference points, with the Euclidean distance as
the closeness measure; the naive method computes every query-point distance.
This module is that naive method, written out.

Fixed readings (the pages leave them open):

* arithmetic is float32, as the points are. The squared distance of query q
  and point p is accumulated dimension by dimension, d = 0, 1, ..., each
  step one rounded product and one rounded sum, with no fused multiply-add:
  ``acc = t0*t0; acc = acc + t1*t1; ...`` with ``td = q[d] - p[d]``;
* neighbours are ordered by (squared distance, original point index), so the
  answer is unique even when distances tie;
* with fewer than K points, the missing entries are index -1 and distance
  +inf.

Coordinates are assumed finite (an infinite one makes differences NaN).
"""
from __future__ import annotations

import numpy as np


def squared_distances(q: np.ndarray, pts: np.ndarray) -> np.ndarray:
    """float32 squared distances of one query q (k,) to every row of pts (n, k)."""
    q = np.asarray(q, dtype=np.float32)
    pts = np.asarray(pts, dtype=np.float32)
    acc = None
    for d in range(pts.shape[1]):
        t = np.float32(q[d]) - pts[:, d]          # float32 - float32 array: rounded
        sq = t * t                                 # rounded product
        acc = sq if acc is None else acc + sq     # rounded sum, dimension order
    if acc is None:
        acc = np.zeros(pts.shape[0], dtype=np.float32)
    return acc.astype(np.float32, copy=False)


def knn_one(q: np.ndarray, pts: np.ndarray, K: int):
    """(indices (K,) int32, squared distances (K,) float32) of query q."""
    n = pts.shape[0]
    idx = np.full(K, -1, dtype=np.int32)
    d2 = np.full(K, np.inf, dtype=np.float32)
    if n == 0 or K == 0:
        return idx, d2
    dist = squared_distances(q, pts)
    take = min(K, n)
    # Every point whose distance is at most the take-th smallest is a
    # candidate (ties included); order the candidates by (distance, index).
    cut = np.partition(dist, take - 1)[take - 1]
    cand = np.nonzero(dist <= cut)[0]
    order = np.lexsort((cand, dist[cand]))[:take]
    idx[:take] = cand[order]
    d2[:take] = dist[cand[order]]
    return idx, d2


def knn(points: np.ndarray, queries: np.ndarray, K: int):
    """Brute-force K nearest neighbours of every query.

    Returns (indices (Q, K) int32, squared distances (Q, K) float32), each row
    ordered by (squared distance, index)."""
    points = np.ascontiguousarray(points, dtype=np.float32)
    queries = np.ascontiguousarray(queries, dtype=np.float32)
    Q = queries.shape[0]
    idx = np.empty((Q, K), dtype=np.int32)
    d2 = np.empty((Q, K), dtype=np.float32)
    for i in range(Q):
        idx[i], d2[i] = knn_one(queries[i], points, K)
    return idx, d2
