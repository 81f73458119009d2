"""Seeded synthetic point sets for the k-d tree build.

This module only draws inputs: it holds none of the build's arithmetic, and
both the GPU path's tests/benchmark and the CPU oracle's tests consume its
arrays. Every generator uses numpy's ``default_rng(seed)`` (PCG64) and returns
a C-contiguous ``(N, k)`` float32 array.

The five named workloads use fixed point counts, dimensions, distributions
and seeds; the pages themselves publish no dataset for
the construction (they quote a "10 million points" build and a 16,777,216 x 4
tuple run), so synthetic data of these shapes stands in.
"""
from __future__ import annotations

import dataclasses
import os

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n: int
    k: int
    dist: str
    seed: int
    note: str


WORKLOADS = {
    "uniform_1k_k3": Workload("uniform_1k_k3", 1000, 3, "uniform", 1,
                              "N=1,000, k=3, U[0,1) float32, seed 1"),
    "uniform_1m_k3": Workload("uniform_1m_k3", 1 << 20, 3, "uniform", 2,
                              "N=1,048,576, k=3, U[0,1) float32, seed 2"),
    "gmm_16m_k3": Workload("gmm_16m_k3", 1 << 24, 3, "gmm", 3,
                           "N=16,777,216, k=3, 64-component isotropic Gaussian mixture "
                           "(centers U[0,1)^3, sigma 0.01), 5% of coordinates snapped to a "
                           "2^-10 grid, seed 3"),
    "normal_4m_k16": Workload("normal_4m_k16", 1 << 22, 16, "normal", 4,
                              "N=4,194,304, k=16, standard normal float32, seed 4"),
    "uniform_100m_k3": Workload("uniform_100m_k3", 100_000_000, 3, "uniform", 5,
                                "N=100,000,000, k=3, U[0,1) float32, seed 5"),
}

# Workload the headline throughput is quoted on.
HEADLINE = "gmm_16m_k3"


def uniform(n: int, k: int, seed: int) -> np.ndarray:
    return default_rng(seed).random((n, k), dtype=np.float32)


def normal(n: int, k: int, seed: int) -> np.ndarray:
    return default_rng(seed).standard_normal((n, k), dtype=np.float32)


def gaussian_mixture(n: int, k: int, seed: int, components: int = 64, sigma: float = 0.01,
                     snap_fraction: float = 0.05, grid: float = 1.0 / 1024) -> np.ndarray:
    """Equal-weight isotropic mixture; computed in float64 and cast once.
    A Bernoulli(snap_fraction) subset of the scalar coordinates is rounded to
    the grid, which forces exact ties (and produces some -0.0 values)."""
    rng = default_rng(seed)
    centers = rng.random((components, k))
    comp = rng.integers(0, components, n)
    x = centers[comp]
    x += sigma * rng.standard_normal((n, k))
    snap = rng.random((n, k)) < snap_fraction
    x[snap] = np.round(x[snap] / grid) * grid
    return np.ascontiguousarray(x.astype(np.float32))


def default_rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def generate(name: str, n: int | None = None) -> np.ndarray:
    """Points of a named workload. A smaller ``n`` redraws with the same recipe
    and seed (for the mixture this is not a prefix of the full-size draw)."""
    w = WORKLOADS[name]
    n = w.n if n is None else int(n)
    if w.dist == "uniform":
        return uniform(n, w.k, w.seed)
    if w.dist == "normal":
        return normal(n, w.k, w.seed)
    if w.dist == "gmm":
        return gaussian_mixture(n, w.k, w.seed)
    raise ValueError(w.dist)


def cached(name: str, cache_dir: str | None = None) -> np.ndarray:
    """generate(name) memoised as .npy (loaded without pickle)."""
    cache_dir = cache_dir or os.environ.get("KDT_DATA_DIR", "/tmp/kdt_data")
    os.makedirs(cache_dir, exist_ok=True)
    path = os.path.join(cache_dir, name + ".npy")
    if os.path.exists(path):
        arr = np.load(path, allow_pickle=False, mmap_mode="r")
        w = WORKLOADS[name]
        if arr.shape == (w.n, w.k) and arr.dtype == np.float32:
            return np.asarray(arr)
    arr = generate(name)
    tmp = path + ".tmp%d.npy" % os.getpid()
    np.save(tmp, arr)
    os.replace(tmp, path)
    return arr


# ---------------------------------------------------------------- edge inputs

def ties(n: int, k: int, seed: int, levels: int = 3) -> np.ndarray:
    """Coordinates drawn from a handful of values: heavy exact ties."""
    rng = default_rng(seed)
    return (rng.integers(0, levels, (n, k)).astype(np.float32) * np.float32(0.5))


def all_equal(n: int, k: int, value: float = 0.25) -> np.ndarray:
    return np.full((n, k), value, dtype=np.float32)


def special_values(n: int, k: int, seed: int) -> np.ndarray:
    """Mix of +-0, +-inf, +-denormals, +-normals and the float extremes."""
    rng = default_rng(seed)
    pool = np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 3e-39, -3e-39,
                     1.0, -1.0, 2.0, -0.5, np.finfo(np.float32).max,
                     -np.finfo(np.float32).max, np.finfo(np.float32).tiny,
                     -np.finfo(np.float32).tiny], dtype=np.float32)
    pick = rng.integers(0, len(pool), (n, k))
    out = pool[pick]
    noise = rng.random((n, k)) < 0.3
    out[noise] = rng.standard_normal(int(noise.sum())).astype(np.float32)
    return np.ascontiguousarray(out)


def signed_zeros(n: int, k: int, seed: int) -> np.ndarray:
    """Only +0.0 and -0.0 (they compare equal, so the index decides)."""
    rng = default_rng(seed)
    return np.where(rng.random((n, k)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
