"""CPU oracle and checker for the left-balanced level-order k-d tree.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``tree_construction_amd``) never imports it, and the two share no code.

Source: I. Wald, "GPU-friendly, Parallel, and (Almost-)In-Place Construction
of Left-Balanced k-d Trees" (arXiv 2211.00120).

* ``build_tree`` -- the recursive builder of ``kdt_oracle.cpp`` (sort the
  subtree's points by (coordinate l mod k, index), take the element whose rank
  equals the left-subtree size, recurse), the builder the paper describes
  before introducing its own method.
* ``check_tree`` -- the independent ancestor-walking checker of
  ``kdt_check.cpp`` (strict k-d condition against every ancestor).
* ``subtree_size`` -- size of a level-order subtree by counting its levels.
* ``brute`` -- exhaustive enumeration for N <= 8 (module ``oracle.brute``).
* ``knn`` -- brute-force K nearest neighbours in float32 (module
  ``oracle.knn``), the reference for the tree's nearest-neighbour query.
* ``build_tree_widest`` -- the split-widest-dimension variant's recursive
  builder (``kdt_widest.cpp``); ``widest_check.check`` verifies such a tree
  by the page's other formulation (domains clipped bottom-up from each node
  to the root).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SOURCES = ("kdt_oracle.cpp", "kdt_check.cpp", "kdt_widest.cpp")
LIB_PATH = os.path.join(_HERE, "libkdt_oracle.so")
_lock = threading.Lock()
_lib = None


def compile_lib(sources_dir: str = _HERE, out_path: str = LIB_PATH, extra_flags=()) -> str:
    """Compile the oracle and checker into one shared library with g++.

    No -ffast-math (IEEE comparisons, denormals kept)."""
    srcs = [os.path.join(sources_dir, s) for s in _SOURCES]
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", *extra_flags,
           "-o", tmp, *srcs]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, out_path)
    return out_path


def _bind(lib):
    lib.kdto_build.restype = ctypes.c_int
    lib.kdto_build.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                               ctypes.c_void_p, ctypes.c_int]
    lib.kdto_subtree_size.restype = ctypes.c_int64
    lib.kdto_subtree_size.argtypes = [ctypes.c_int64, ctypes.c_int64]
    lib.kdto_check.restype = ctypes.c_int64
    lib.kdto_check.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
    lib.kdto_build_widest.restype = ctypes.c_int
    lib.kdto_build_widest.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.kdto_max_threads.restype = ctypes.c_int
    lib.kdto_max_threads.argtypes = []
    return lib


def load_lib(path: str | None = None):
    """Load the oracle library, compiling it first if it is missing or stale."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            newest_src = max(os.path.getmtime(os.path.join(_HERE, s)) for s in _SOURCES)
            if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < newest_src:
                compile_lib()
            _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _points(points) -> np.ndarray:
    pts = np.ascontiguousarray(points, dtype=np.float32)
    if pts.ndim != 2:
        raise ValueError("points must be an (N, k) array")
    return pts


def build_tree(points, nthreads: int = 0, lib=None) -> np.ndarray:
    """Level-order permutation: perm[node] = original index of its point."""
    lib = lib or load_lib()
    pts = _points(points)
    n, k = pts.shape
    perm = np.empty(n, dtype=np.int32)
    rc = lib.kdto_build(pts.ctypes.data, n, k, perm.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected arguments (N=%d, k=%d)" % (n, k))
    return perm


def build_tree_widest(points, nthreads: int = 0, lib=None):
    """Split-widest-dimension tree (kdt_widest.cpp): (perm, dims), perm[node]
    = original index of its point, dims[node] = its split dimension."""
    lib = lib or load_lib()
    pts = _points(points)
    n, k = pts.shape
    perm = np.empty(n, dtype=np.int32)
    dims = np.empty(n, dtype=np.int32)
    rc = lib.kdto_build_widest(pts.ctypes.data, n, k, perm.ctypes.data, dims.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected arguments (N=%d, k=%d)" % (n, k))
    return perm, dims


def check_tree(points, perm, lib=None) -> int:
    """-1 when perm is the tree; else the first offending node (N + slot for a
    non-permutation)."""
    lib = lib or load_lib()
    pts = _points(points)
    n, k = pts.shape
    p = np.ascontiguousarray(perm, dtype=np.int32)
    if p.shape != (n,):
        raise ValueError("perm must have N entries")
    return int(lib.kdto_check(pts.ctypes.data, n, k, p.ctypes.data))


def subtree_size(N: int, c: int, lib=None) -> int:
    lib = lib or load_lib()
    return int(lib.kdto_subtree_size(int(N), int(c)))


def max_threads(lib=None) -> int:
    lib = lib or load_lib()
    return int(lib.kdto_max_threads())
