"""GPU parity of the K-nearest-neighbour query (kdt_knn through the C ABI)
against the brute-force float32 oracle (oracle/knn.py).

Indices and squared distances must be bit-identical: the query ranks by
(float32 squared distance, original index) exactly as brute force does.
Cases cover empty and tiny trees, K above N (padding), heavy distance ties
(few distinct coordinates, all-equal points, signed zeros), queries equal to
tree points, k from 1 to 16, every K bucket up to 32, ragged query counts,
and the headline 16M-point workload on sampled queries.
"""
import sys

import numpy as np
import pytest

from oracle import knn as knn_oracle
from tree_construction_amd import datagen, kdt

pytestmark = pytest.mark.gpu


def say(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    return torch, torch.device("cuda:0")


def gpu_knn(torch_dev, pts, qs, K):
    torch, dev = torch_dev
    x = torch.from_numpy(np.ascontiguousarray(pts)).to(dev)
    q = torch.from_numpy(np.ascontiguousarray(qs)).to(dev)
    if len(pts):
        perm, tree = kdt.build(x)
    else:
        perm, tree = None, None
    idx, d2 = kdt.knn(tree, perm, q, K)
    torch.cuda.synchronize(dev)
    return idx.cpu().numpy(), d2.cpu().numpy()


def assert_same(pts, qs, K, idx, d2, label):
    want_idx, want_d2 = knn_oracle.knn(pts, qs, K)
    if not np.array_equal(idx, want_idx):
        r = int(np.flatnonzero((idx != want_idx).any(1))[0])
        raise AssertionError("%s: query %d gpu %s oracle %s" % (label, r, idx[r].tolist(), want_idx[r].tolist()))
    assert np.array_equal(d2.view(np.uint32), want_d2.view(np.uint32)), label


def make(gen, n, k, seed):
    if gen == "uniform":
        return datagen.uniform(n, k, seed)
    if gen == "gmm":
        return datagen.gaussian_mixture(n, k, seed)
    if gen == "ties":
        return datagen.ties(n, k, seed)
    if gen == "equal":
        return datagen.all_equal(n, k)
    if gen == "zeros":
        return datagen.signed_zeros(n, k, seed)
    if gen == "normal":
        return datagen.normal(n, k, seed)
    raise ValueError(gen)


@pytest.mark.parametrize("gen", ["uniform", "gmm", "ties", "equal", "zeros", "normal"])
def test_knn_sizes(torch_dev, gen):
    rng = np.random.default_rng(5)
    for i, n in enumerate([1, 2, 3, 7, 31, 100, 1000, 4097, 20011]):
        k = (1, 2, 3, 4, 5, 16)[i % 6]
        K = (1, 2, 3, 5, 8, 13, 16, 25, 32)[i % 9]
        pts = make(gen, n, k, 40 + i)
        q = int(rng.integers(1, 300))
        qs = make(gen if gen not in ("equal",) else "uniform", q, k, 900 + i)
        # some queries sit exactly on tree points
        hit = rng.integers(0, n, max(1, q // 4))
        qs[: len(hit)] = pts[hit]
        say("case knn gen=%s N=%d k=%d K=%d Q=%d" % (gen, n, k, K, q))
        idx, d2 = gpu_knn(torch_dev, pts, qs, K)
        assert_same(pts, qs, K, idx, d2, "%s N=%d k=%d K=%d" % (gen, n, k, K))


@pytest.mark.parametrize("budget", [0, 1, 37])
def test_knn_wave_pass(torch_dev, budget):
    """Small first-pass budgets hand (nearly) every query to the wave pass."""
    torch, dev = torch_dev
    rng = np.random.default_rng(budget + 3)
    cases = [("gmm", 30000, 3, 8), ("ties", 5000, 3, 5), ("uniform", 4097, 2, 32), ("normal", 3000, 5, 16),
             ("zeros", 2000, 4, 3), ("equal", 700, 3, 9), ("uniform", 5, 3, 8), ("gmm", 200000, 3, 1)]
    for gen, n, k, K in cases:
        pts = make(gen, n, k, 70 + n % 13)
        qs = make(gen if gen != "equal" else "uniform", 333, k, 71)
        qs[:50] = pts[rng.integers(0, n, 50)]
        x = torch.from_numpy(pts).to(dev)
        perm, tree = kdt.build(x)
        visits = torch.empty(len(qs), dtype=torch.int32, device=dev)
        say("case knn wave budget=%d gen=%s N=%d k=%d K=%d" % (budget, gen, n, k, K))
        idx, d2 = kdt.knn(tree, perm, torch.from_numpy(qs).to(dev), K, visits=visits, budget=budget)
        torch.cuda.synchronize(dev)
        assert_same(pts, qs, K, idx.cpu().numpy(), d2.cpu().numpy(), "wave budget=%d %s" % (budget, gen))
        v = visits.cpu().numpy()
        assert (v >= 1).all() and (v <= n + budget).all()


@pytest.mark.parametrize("budget", [None, 0])
def test_knn_split_widest_tree(torch_dev, budget):
    """Over a split-widest tree (per-node dimensions) the answers are the same
    brute-force ones."""
    torch, dev = torch_dev
    for gen, n, k, K in [("gmm", 40000, 3, 8), ("ties", 3000, 2, 5), ("uniform", 4097, 4, 32),
                         ("normal", 2500, 5, 3), ("zeros", 1000, 3, 7)]:
        pts = make(gen, n, k, 500 + n % 7)
        qs = make(gen, 300, k, 501)
        qs[:30] = pts[:30]
        x = torch.from_numpy(pts).to(dev)
        perm, tree, dims = kdt.build_widest(x)
        say("case knn widest budget=%s gen=%s N=%d k=%d K=%d" % (budget, gen, n, k, K))
        idx, d2 = kdt.knn(tree, perm, torch.from_numpy(qs).to(dev), K, dims=dims, budget=budget)
        torch.cuda.synchronize(dev)
        assert_same(pts, qs, K, idx.cpu().numpy(), d2.cpu().numpy(), "widest %s" % gen)


def test_knn_every_k_bucket(torch_dev):
    pts = datagen.gaussian_mixture(50000, 3, 8)
    qs = datagen.gaussian_mixture(777, 3, 8)  # same centres, other draws
    for K in range(1, 33):
        say("case knn bucket K=%d" % K)
        idx, d2 = gpu_knn(torch_dev, pts, qs, K)
        assert_same(pts, qs, K, idx, d2, "K=%d" % K)


def test_knn_empty_tree_and_no_queries(torch_dev):
    torch, dev = torch_dev
    qs = datagen.uniform(5, 3, 1)
    say("case knn empty tree")
    idx, d2 = gpu_knn(torch_dev, np.zeros((0, 3), np.float32), qs, 4)
    assert (idx == -1).all() and np.isinf(d2).all()
    say("case knn no queries")
    idx, d2 = gpu_knn(torch_dev, datagen.uniform(10, 3, 2), np.zeros((0, 3), np.float32), 4)
    assert idx.shape == (0, 4)


def test_knn_visits(torch_dev):
    torch, dev = torch_dev
    pts = datagen.uniform(3000, 3, 21)
    x = torch.from_numpy(pts).to(dev)
    perm, tree = kdt.build(x)
    q = torch.from_numpy(datagen.uniform(500, 3, 22)).to(dev)
    visits = torch.empty(500, dtype=torch.int32, device=dev)
    say("case knn visits")
    kdt.knn(tree, perm, q, 8, visits=visits)
    v = visits.cpu().numpy()
    assert (v >= 1).all() and (v <= 3000).all() and v.mean() < 3000
    # a search that never fills its K slots cannot prune: it examines every point
    small = x[:20].contiguous()
    perm_s, tree_s = kdt.build(small)
    kdt.knn(tree_s, perm_s, q, 32, visits=visits)
    assert (visits.cpu().numpy() == 20).all()


def test_knn_rejects_bad_arguments(torch_dev):
    torch, dev = torch_dev
    pts = torch.from_numpy(datagen.uniform(100, 3, 3)).to(dev)
    perm, tree = kdt.build(pts)
    for K in (0, 33):
        with pytest.raises(kdt.KdtError):
            kdt.knn(tree, perm, pts, K)


def default_budget(K):
    """The first pass's hand-over budget of kdt_knn: 32 K within [128, 512]."""
    return min(max(32 * K, 128), 512)


@pytest.mark.parametrize("K", [8, 32])
def test_knn_headline_workload_sampled(torch_dev, K):
    torch, dev = torch_dev
    name = datagen.HEADLINE
    pts = datagen.cached(name)
    qs = datagen.generate(name, n=1 << 20)  # the workload's recipe, other draws
    x = torch.from_numpy(pts).to(dev)
    q = torch.from_numpy(qs).to(dev)
    perm, tree = kdt.build(x)
    say("case knn %s Q=%d K=%d" % (name, len(qs), K))
    visits = torch.empty(len(qs), dtype=torch.int32, device=dev)
    idx, d2 = kdt.knn(tree, perm, q, K, visits=visits)
    torch.cuda.synchronize(dev)
    idx, d2, v = idx.cpu().numpy(), d2.cpu().numpy(), visits.cpu().numpy()
    # the 100 most expensive searches (the first pass hands them to the wave
    # pass: more than its budget of points examined), 256 random ones, and
    # the first and last query
    costly = np.argsort(-v.astype(np.int64), kind="stable")[:100]
    assert v[costly[-1]] > default_budget(K), "the sample must include wave-pass queries"
    rng = np.random.default_rng(17)
    sample = np.unique(np.concatenate([costly, rng.choice(len(qs), 256, replace=False), [0, len(qs) - 1]]))
    say("  checking %d queries against brute force" % len(sample))
    want_idx, want_d2 = knn_oracle.knn(pts, qs[sample], K)
    assert np.array_equal(idx[sample], want_idx)
    assert np.array_equal(d2[sample].view(np.uint32), want_d2.view(np.uint32))


@pytest.mark.parametrize("gen,cap", [("equal", 1), ("equal", 64), ("gmm", 1), ("gmm", 100), ("ties", 7)])
def test_knn_wave_stack_overflow(torch_dev, gen, cap):
    """With the wave pass's stack capped, the far sides that do not fit are
    walked by their lanes alone (the path a full stack takes); the answer is
    still brute force's. Identical points never prune (a far side is skipped
    only when strictly farther than the K-th distance): every point is
    examined."""
    torch, dev = torch_dev
    n = 50000
    pts = {"equal": lambda: datagen.all_equal(n, 3), "gmm": lambda: datagen.gaussian_mixture(n, 3, 5),
           "ties": lambda: datagen.ties(n, 3, 6)}[gen]()
    x = torch.from_numpy(pts).to(dev)
    perm, tree = kdt.build(x)
    qs = np.concatenate([pts[:8], datagen.uniform(56, 3, 41)]).astype(np.float32)
    q = torch.from_numpy(qs).to(dev)
    for K in (1, 8, 32):
        say("case knn wave stack cap=%d %s N=%d K=%d budget=0" % (cap, gen, n, K))
        visits = torch.empty(len(qs), dtype=torch.int32, device=dev)
        idx, d2 = kdt.knn(tree, perm, q, K, visits=visits, budget=0, wave_stack=cap)
        torch.cuda.synchronize(dev)
        want_idx, want_d2 = knn_oracle.knn(pts, qs, K)
        assert np.array_equal(idx.cpu().numpy(), want_idx)
        assert np.array_equal(d2.cpu().numpy().view(np.uint32), want_d2.view(np.uint32))
        if gen == "equal":
            assert (visits.cpu().numpy() == n).all()


def test_knn_wave_stack_cap_rejected(torch_dev):
    torch, dev = torch_dev
    pts = torch.from_numpy(datagen.uniform(100, 3, 3)).to(dev)
    perm, tree = kdt.build(pts)
    for cap in (0, 2049):
        with pytest.raises(kdt.KdtError):
            kdt.knn(tree, perm, pts, 4, wave_stack=cap)
