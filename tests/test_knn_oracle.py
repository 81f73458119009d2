"""Pins for the brute-force k-nearest-neighbour oracle (oracle/knn.py); no GPU.

The oracle is the naive search of F. Gieseke et al., "Bigger Buffer k-d Trees
on Multi-Many-Core Systems" (arXiv 1512.02831), section 2.3 and the problem
statement before it. It is checked against things other than itself:

* hand-derived answers on integer points (tests/golden/knn_hand_example.txt);
* scipy's k-d tree query in float64 (a library routine): the neighbour sets
  agree up to float32 rounding of the distances;
* exact integer arithmetic in Python for K >= N (the whole ranking) and for
  one-dimensional data;
* identical points: the index tie-break alone orders them;
* a hand-derived float32 case where rounding (and the order of the sum)
  decides the ranking.

test_planted_mistakes_are_caught runs plausible wrong variants of the oracle
through the same pins and requires each to fail at least one.
"""
import math
import os

import numpy as np
import pytest

from oracle import knn as knn_oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def load_hand_example():
    pts, cases, cur = [], [], None
    with open(os.path.join(HERE, "golden", "knn_hand_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, *vals = line.split()
            if tag == "point":
                pts.append([float(v) for v in vals])
            elif tag == "query":
                cur = {"q": [float(v) for v in vals]}
                cases.append(cur)
            elif tag == "K":
                cur["K"] = int(vals[0])
            elif tag == "idx":
                cur["idx"] = [int(v) for v in vals]
            elif tag == "d2":
                cur["d2"] = [float(v) for v in vals]
    return np.array(pts, dtype=np.float32), cases


# ------------------------------------------------------------------- pins
# Each returns None when the given knn function passes, else a message.

def pin_hand_example(fn):
    pts, cases = load_hand_example()
    for c in cases:
        idx, d2 = fn(pts, np.array([c["q"]], dtype=np.float32), c["K"])
        if idx[0].tolist() != c["idx"] or d2[0].tolist() != c["d2"]:
            return "hand example %s: %s %s" % (c["q"], idx[0].tolist(), d2[0].tolist())
    return None


def pin_scipy(fn):
    from scipy.spatial import cKDTree
    rng = np.random.default_rng(7)
    pts = rng.random((3000, 3), dtype=np.float32)
    qs = rng.random((40, 3), dtype=np.float32)
    K = 8
    ref_d, _ = cKDTree(pts.astype(np.float64)).query(qs.astype(np.float64), K)
    idx, d2 = fn(pts, qs, K)
    for i in range(len(qs)):
        got = np.sqrt(((pts[idx[i]].astype(np.float64) - qs[i].astype(np.float64)) ** 2).sum(1))
        # float32 distances may reorder neighbours only within rounding
        if not np.allclose(np.sort(got), ref_d[i], rtol=1e-5, atol=1e-7):
            return "query %d: %s vs %s" % (i, got, ref_d[i])
        if not np.allclose(np.sqrt(d2[i].astype(np.float64)), ref_d[i], rtol=1e-5, atol=1e-7):
            return "query %d distances %s vs %s" % (i, d2[i], ref_d[i])
    return None


def pin_exact_integer_ranking(fn):
    rng = np.random.default_rng(11)
    for k in (1, 2, 3, 5):
        pts = rng.integers(-20, 21, (37, k))
        qs = rng.integers(-25, 26, (6, k))
        K = 45  # more than N: the whole ranking plus padding
        idx, d2 = fn(pts.astype(np.float32), qs.astype(np.float32), K)
        for i, q in enumerate(qs.tolist()):
            exact = sorted((sum((a - b) ** 2 for a, b in zip(q, p)), j) for j, p in enumerate(pts.tolist()))
            want_idx = [j for _, j in exact] + [-1] * (K - len(exact))
            want_d2 = [float(d) for d, _ in exact] + [math.inf] * (K - len(exact))
            if idx[i].tolist() != want_idx or d2[i].tolist() != want_d2:
                return "k=%d query %d" % (k, i)
    return None


def pin_identical_points(fn):
    pts = np.full((20, 3), 0.5, dtype=np.float32)
    idx, d2 = fn(pts, np.array([[0.0, 1.0, 0.25]], dtype=np.float32), 7)
    if idx[0].tolist() != list(range(7)) or len(set(d2[0].tolist())) != 1:
        return "identical points: %s" % idx[0].tolist()
    return None


def pin_float32_rounding():
    """Hand-derived float32 case. Query at the origin; points
    A = (1, 2^-12, 0), B = (1, 0, 0), C = (1, 2^-12, 2^-12) (indices 0, 1, 2).
    Exact squared distances: A 1 + 2^-24, B 1, C 1 + 2^-23. In float32 with
    dimension-order accumulation: A = 1 + 2^-24 rounds (half-way, to even) to
    1; C = (1 + 2^-24) + 2^-24 -> 1 then 1 again. All three are 1.0, so the
    index orders them: [0, 1, 2] with distances [1, 1, 1]. (float64 would give
    [1, 0, 2]; summing the other way round would give C 1 + 2^-23.)"""
    def check(fn):
        e = np.float32(2.0 ** -12)
        pts = np.array([[1, e, 0], [1, 0, 0], [1, e, e]], dtype=np.float32)
        idx, d2 = fn(pts, np.zeros((1, 3), dtype=np.float32), 3)
        if idx[0].tolist() != [0, 1, 2] or d2[0].tolist() != [1.0, 1.0, 1.0]:
            return "float32 rounding: %s %s" % (idx[0].tolist(), d2[0].tolist())
        return None
    check.__name__ = "pin_float32_rounding"
    return check


PINS = [pin_hand_example, pin_scipy, pin_exact_integer_ranking, pin_identical_points, pin_float32_rounding()]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pins(pin):
    assert pin(knn_oracle.knn) is None


def test_rows_are_ordered_and_distances_recompute():
    rng = np.random.default_rng(3)
    pts = rng.normal(size=(500, 4)).astype(np.float32)
    qs = rng.normal(size=(20, 4)).astype(np.float32)
    idx, d2 = knn_oracle.knn(pts, qs, 12)
    for i in range(len(qs)):
        assert len(set(idx[i].tolist())) == 12
        keys = list(zip(d2[i].tolist(), idx[i].tolist()))
        assert keys == sorted(keys)
        np.testing.assert_array_equal(d2[i], knn_oracle.squared_distances(qs[i], pts)[idx[i]])


# ------------------------------------------------------ planted mistakes

def _variant(mistake):
    def squared(q, pts):
        q = np.asarray(q, dtype=np.float32)
        dims = range(pts.shape[1] - 1) if mistake == "drop_last_dim" and pts.shape[1] > 1 else range(pts.shape[1])
        acc = np.zeros(pts.shape[0], dtype=np.float64 if mistake == "float64" else np.float32)
        if mistake == "reverse_dim_order":
            dims = reversed(list(dims))
        for d in dims:
            t = (q[d].astype(acc.dtype) - pts[:, d].astype(acc.dtype))
            acc = acc + (np.abs(t) if mistake == "abs_not_square" else t * t)
        return acc.astype(np.float32)

    def fn(points, queries, K):
        points = np.asarray(points, dtype=np.float32)
        Q, n = len(queries), len(points)
        idx = np.full((Q, K), -1, dtype=np.int32)
        d2 = np.full((Q, K), np.inf, dtype=np.float32)
        for i in range(Q):
            dist = squared(queries[i], points)
            ids = np.arange(n)
            tie = -ids if mistake == "tie_by_larger_index" else ids
            order = np.lexsort((tie, dist))[:min(K, n)]
            if mistake == "no_padding":
                order = order[:K]
                idx[i, :len(order)] = order
                d2[i, :len(order)] = dist[order]
                idx[i, len(order):] = 0
                d2[i, len(order):] = 0
                continue
            idx[i, :len(order)] = order
            d2[i, :len(order)] = dist[order]
        return idx, d2
    return fn


@pytest.mark.parametrize("mistake", ["drop_last_dim", "float64", "abs_not_square", "tie_by_larger_index",
                                     "no_padding", "reverse_dim_order"])
def test_planted_mistakes_are_caught(mistake):
    fn = _variant(mistake)
    failed = [p.__name__ for p in PINS if p(fn) is not None]
    assert failed, "no pin caught %s" % mistake


def test_correct_variant_passes_all_pins():
    # the mutation harness itself is sound: with no mistake every pin passes
    fn = _variant(None)
    assert [p.__name__ for p in PINS if p(fn) is not None] == []
