"""Builds captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

A build enqueues kernels only: no allocation, copy, memset or host
synchronisation, so a caller can capture it once per workspace and replay it
with new coordinates in the same buffers. Each graph is replayed several
times, with eager work on the same stream between the replays (the outputs
cleared, the points rewritten), and every replay is checked against the
oracle for the points it saw.
"""
import sys

import numpy as np
import pytest

import oracle
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


def capture(torch, fn):
    """Warm up on a side stream, as graph capture wants, then capture fn."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


# (N, k): array rounds and the LDS record stage (k = 3), per-point tag rounds
# and the columns stage (k = 16), one subtree from the rows (N <= 4096)
@pytest.mark.parametrize("n,k", [(300000, 3), (300000, 16), (3000, 5)])
def test_build_graph_replays(torch_dev, n, k):
    torch, dev = torch_dev
    inputs = [datagen.gaussian_mixture(n, k, 40 + r) if r % 2 == 0 else datagen.ties(n, k, 40 + r)
              for r in range(3)]
    x = torch.from_numpy(np.ascontiguousarray(inputs[0])).to(dev)
    b = kdt.Builder(n, k, dev)
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    tree = torch.empty_like(x)
    say("case graph build N=%d k=%d" % (n, k))
    graph = capture(torch, lambda: b.build(x, perm, tree))
    for r, pts in enumerate(inputs):
        x.copy_(torch.from_numpy(np.ascontiguousarray(pts)))
        perm.fill_(-1)
        tree.zero_()
        graph.replay()
        torch.cuda.synchronize()
        want = oracle.build_tree(pts)
        got = perm.cpu().numpy()
        assert np.array_equal(got, want), "replay %d: %d nodes differ" % (r, int((got != want).sum()))
        assert np.array_equal(tree.cpu().numpy().view(np.uint32), pts[want].view(np.uint32)), "replay %d" % r


@pytest.mark.parametrize("n,k", [(300000, 3), (300000, 8)])
def test_widest_graph_replays(torch_dev, n, k):
    torch, dev = torch_dev
    inputs = [datagen.gaussian_mixture(n, k, 60 + r) for r in range(3)]
    x = torch.from_numpy(np.ascontiguousarray(inputs[0])).to(dev)
    b = kdt.WidestBuilder(n, k, dev)
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    tree = torch.empty_like(x)
    dims = torch.empty(n, dtype=torch.int32, device=dev)
    say("case graph widest N=%d k=%d" % (n, k))
    graph = capture(torch, lambda: b.build(x, perm, tree, dims))
    for r, pts in enumerate(inputs):
        x.copy_(torch.from_numpy(np.ascontiguousarray(pts)))
        perm.fill_(-1)
        dims.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        want_p, want_d = oracle.build_tree_widest(pts)
        assert np.array_equal(perm.cpu().numpy(), want_p), "replay %d" % r
        assert np.array_equal(dims.cpu().numpy(), want_d), "replay %d" % r
        assert np.array_equal(tree.cpu().numpy().view(np.uint32), pts[want_p].view(np.uint32)), "replay %d" % r
