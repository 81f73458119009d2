"""Python binding of the C ABI in include/kdt.h (ctypes; argument marshalling only).

Every step of the build runs in libkdt.so's HIP kernels; this module only
allocates device buffers with torch, passes raw pointers and the current HIP
stream, and turns status codes into exceptions. If libkdt.so is missing the
import-time load fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkdt.so")

KDT_OK = 0
STATUS_NAMES = {0: "KDT_OK", 1: "KDT_ERR_INVALID_ARG", 2: "KDT_ERR_WORKSPACE", 3: "KDT_ERR_HIP",
                4: "KDT_ERR_TOO_LARGE"}
STATIC_SCRATCH_BYTES = 64 << 20  # KDT_STATIC_SCRATCH_BYTES

PROFILE_MAX_KINDS = 32
PROFILE_NAME_LEN = 48


class Profile(ctypes.Structure):
    """Mirror of kdt_profile."""
    _fields_ = [("kinds", ctypes.c_int32),
                ("name", (ctypes.c_char * PROFILE_NAME_LEN) * PROFILE_MAX_KINDS),
                ("launches", ctypes.c_int64 * PROFILE_MAX_KINDS),
                ("ms", ctypes.c_double * PROFILE_MAX_KINDS),
                ("bytes", ctypes.c_double * PROFILE_MAX_KINDS)]

    def as_dict(self):
        return {self.name[i].value.decode(): {"launches": int(self.launches[i]),
                                              "ms": float(self.ms[i]),
                                              "bytes": float(self.bytes[i])}
                for i in range(self.kinds)}


# Every function include/kdt.h declares: name -> (restype, argtypes).
_VOIDP, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
SIGNATURES = {
    "kdt_workspace_size": (_SZ, [_I64, _I32]),
    "kdt_build": (ctypes.c_int, [_VOIDP, _I64, _I32, _VOIDP, _VOIDP, _VOIDP, _SZ, _VOIDP]),
    "kdt_build_static": (ctypes.c_int, [_VOIDP, _I64, _I32, _VOIDP, _VOIDP, _VOIDP]),
    "kdt_debug_tags": (ctypes.c_int, [_VOIDP, _I64, _I32, _I32, _VOIDP, _VOIDP, _SZ, _VOIDP]),
    "kdt_build_profiled": (ctypes.c_int, [_VOIDP, _I64, _I32, _VOIDP, _VOIDP, _VOIDP, _SZ, _VOIDP,
                                          ctypes.POINTER(Profile)]),
    "kdt_closed_subtree_size": (_I64, [_I64, _I64]),
    "kdt_closed_segment_begin": (_I64, [_I64, _I64, _I32]),
    "kdt_debug_workspace_size": (_SZ, [_I64, _I32, _I32]),
    "kdt_closed_live_segment": (_I64, [_I64, _I32, _I64]),
    "kdt_closed_bin_prefix": (_I64, [_I64, _I32, _I32, _I64, _I64]),
    "kdt_closed_float_keys": (None, [_VOIDP, _I64, _VOIDP]),
    "kdt_knn": (ctypes.c_int, [_VOIDP, _VOIDP, _VOIDP, _I64, _I32, _VOIDP, _I64, _I32, _VOIDP, _VOIDP, _VOIDP,
                               _VOIDP]),
    "kdt_knn_budget": (ctypes.c_int, [_VOIDP, _VOIDP, _VOIDP, _I64, _I32, _VOIDP, _I64, _I32, _VOIDP, _VOIDP,
                                      _VOIDP, ctypes.c_uint32, _VOIDP]),
    "kdt_knn_debug": (ctypes.c_int, [_VOIDP, _VOIDP, _VOIDP, _I64, _I32, _VOIDP, _I64, _I32, _VOIDP, _VOIDP,
                                     _VOIDP, ctypes.c_uint32, ctypes.c_uint32, _VOIDP]),
    "kdt_unique_workspace_size": (_SZ, [_I64, _I32]),
    "kdt_unique": (ctypes.c_int, [_VOIDP, _I64, _I32, _VOIDP, _VOIDP, _VOIDP, _SZ, _VOIDP]),
    "kdt_unique_profiled": (ctypes.c_int, [_VOIDP, _I64, _I32, _VOIDP, _VOIDP, _VOIDP, _SZ, _VOIDP,
                                           ctypes.POINTER(Profile)]),
    "kdt_workspace_size_widest": (_SZ, [_I64, _I32]),
    "kdt_build_widest": (ctypes.c_int, [_VOIDP, _I64, _I32, _VOIDP, _VOIDP, _VOIDP, _VOIDP, _SZ, _VOIDP]),
    "kdt_build_widest_profiled": (ctypes.c_int, [_VOIDP, _I64, _I32, _VOIDP, _VOIDP, _VOIDP, _VOIDP, _SZ,
                                                 _VOIDP, ctypes.POINTER(Profile)]),
    "kdt_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

KNN_MAX_K = 32

_lock = threading.Lock()
_lib = None


class KdtError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, STATUS_NAMES.get(status, status),
                                          lib().kdt_status_string(status).decode()))


def lib():
    """The loaded libkdt.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libkdt.so not built: run __graft_entry__.build() "
                                   "or python -m tree_construction_amd.build_lib")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def workspace_size(n: int, k: int) -> int:
    return int(lib().kdt_workspace_size(int(n), int(k)))


def closed_subtree_size(n: int, s: int) -> int:
    return int(lib().kdt_closed_subtree_size(int(n), int(s)))


def closed_segment_begin(n: int, s: int, level: int) -> int:
    return int(lib().kdt_closed_segment_begin(int(n), int(s), int(level)))


def debug_workspace_size(n: int, k: int, rounds: int) -> int:
    return int(lib().kdt_debug_workspace_size(int(n), int(k), int(rounds)))


def closed_live_segment(n: int, level: int, p: int) -> int:
    return int(lib().kdt_closed_live_segment(int(n), int(level), int(p)))


def closed_bin_prefix(n: int, l1: int, delta: int, j0: int, b: int) -> int:
    return int(lib().kdt_closed_bin_prefix(int(n), int(l1), int(delta), int(j0), int(b)))


def closed_float_keys(bits):
    """Keys of float32 bit patterns (a uint32 numpy array), computed by the
    library's host copy of the kernels' key transform."""
    import numpy as np
    b = np.ascontiguousarray(bits, dtype=np.uint32)
    out = np.empty_like(b)
    lib().kdt_closed_float_keys(b.ctypes.data, b.size, out.ctypes.data)
    return out


def _check(status: int, where: str):
    if status != KDT_OK:
        raise KdtError(status, where)


def _stream_handle(device, stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _used_on(stream, device, *tensors):
    """Mark tensors that kernels enqueued on `stream` use, when that stream is
    not the current one: the caching allocator then keeps their memory until
    that work is done, even if the tensors are freed earlier."""
    import torch
    if stream is None or stream == torch.cuda.current_stream(device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _validate_points(points):
    import torch
    if not isinstance(points, torch.Tensor) or points.dtype != torch.float32 or points.dim() != 2:
        raise TypeError("points must be a 2-D float32 torch tensor")
    if not points.is_cuda:
        raise ValueError("points must be on a HIP device")
    if not points.is_contiguous():
        raise ValueError("points must be contiguous (row-major N x k)")


class Builder:
    """Holds a workspace sized for (N, k) so repeated builds allocate nothing."""

    def __init__(self, n: int, k: int, device="cuda"):
        import torch
        self.n, self.k = int(n), int(k)
        self.device = torch.device(device)
        nbytes = workspace_size(self.n, self.k)
        if nbytes == 0 and self.n > 1:
            raise ValueError("unsupported size N=%d k=%d" % (self.n, self.k))
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)
        self.workspace_bytes = nbytes

    def build(self, points, perm=None, tree=None, want_tree=True, stream=None):
        import torch
        _validate_points(points)
        if tuple(points.shape) != (self.n, self.k):
            raise ValueError("points shape %s != (%d, %d)" % (tuple(points.shape), self.n, self.k))
        if perm is None:
            perm = torch.empty(self.n, dtype=torch.int32, device=points.device)
        if tree is None and want_tree:
            tree = torch.empty_like(points)
        st = lib().kdt_build(ctypes.c_void_p(points.data_ptr()), self.n, self.k,
                             ctypes.c_void_p(perm.data_ptr()),
                             ctypes.c_void_p(tree.data_ptr() if tree is not None else 0),
                             ctypes.c_void_p(self.workspace.data_ptr()), self.workspace_bytes,
                             _stream_handle(points.device, stream))
        _check(st, "kdt_build")
        _used_on(stream, points.device, self.workspace, points, perm, tree)
        return perm, tree

    def build_profiled(self, points, perm, tree=None, stream=None):
        """One build with a HIP event pair around every kernel; synchronises
        and returns {kernel kind: {launches, ms, bytes}}."""
        _validate_points(points)
        prof = Profile()
        st = lib().kdt_build_profiled(ctypes.c_void_p(points.data_ptr()), self.n, self.k,
                                      ctypes.c_void_p(perm.data_ptr()),
                                      ctypes.c_void_p(tree.data_ptr() if tree is not None else 0),
                                      ctypes.c_void_p(self.workspace.data_ptr()),
                                      self.workspace_bytes, _stream_handle(points.device, stream),
                                      ctypes.byref(prof))
        _check(st, "kdt_build_profiled")
        return prof.as_dict()

    def debug_tags(self, points, rounds: int, stream=None):
        """int32 tensor holding the uint32 tags after `rounds` rounds (uses a
        workspace of its own, sized by kdt_debug_workspace_size)."""
        import torch
        _validate_points(points)
        out = torch.empty(self.n, dtype=torch.int32, device=points.device)
        nbytes = debug_workspace_size(self.n, self.k, rounds)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=points.device)
        st = lib().kdt_debug_tags(ctypes.c_void_p(points.data_ptr()), self.n, self.k, int(rounds),
                                  ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                  nbytes, _stream_handle(points.device, stream))
        _check(st, "kdt_debug_tags")
        _used_on(stream, points.device, ws, points, out)
        return out


def unique_workspace_size(n: int, k: int) -> int:
    return int(lib().kdt_unique_workspace_size(int(n), int(k)))


class UniqueFinder:
    """Duplicate removal for (N, k) points with a held workspace."""

    def __init__(self, n: int, k: int, device="cuda"):
        import torch
        self.n, self.k = int(n), int(k)
        self.device = torch.device(device)
        nbytes = unique_workspace_size(self.n, self.k)
        if nbytes == 0 and self.n > 0:
            raise ValueError("unsupported size N=%d k=%d" % (self.n, self.k))
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)
        self.workspace_bytes = nbytes
        self.count = torch.empty(1, dtype=torch.int64, device=self.device)

    def _args(self, points, keep, stream):
        return (ctypes.c_void_p(points.data_ptr()), self.n, self.k, ctypes.c_void_p(keep.data_ptr()),
                ctypes.c_void_p(self.count.data_ptr()), ctypes.c_void_p(self.workspace.data_ptr()),
                self.workspace_bytes, _stream_handle(points.device, stream))

    def run(self, points, keep=None, stream=None):
        """Enqueue; returns (keep, count) with count a 1-element device tensor."""
        import torch
        _validate_points(points)
        if tuple(points.shape) != (self.n, self.k):
            raise ValueError("points shape %s != (%d, %d)" % (tuple(points.shape), self.n, self.k))
        if keep is None:
            keep = torch.empty(max(self.n, 1), dtype=torch.int32, device=points.device)
        _check(lib().kdt_unique(*self._args(points, keep, stream)), "kdt_unique")
        _used_on(stream, points.device, self.workspace, self.count, points, keep)
        return keep, self.count

    def run_profiled(self, points, keep, stream=None):
        _validate_points(points)
        prof = Profile()
        _check(lib().kdt_unique_profiled(*self._args(points, keep, stream), ctypes.byref(prof)),
               "kdt_unique_profiled")
        return prof.as_dict()


def unique(points, stream=None):
    """Ascending original indices of one point (the smallest index) of every
    distinct tuple of `points` ((N, k) float32 on a HIP device): an int32
    device tensor (synchronises to read the count)."""
    import torch
    _validate_points(points)
    n, k = points.shape
    keep, count = UniqueFinder(n, k, points.device).run(points, stream=stream)
    # the count is written on `stream`: wait for that stream, not the current one
    (stream if stream is not None else torch.cuda.current_stream(points.device)).synchronize()
    return keep[: int(count.item())]


def workspace_size_widest(n: int, k: int) -> int:
    return int(lib().kdt_workspace_size_widest(int(n), int(k)))


class WidestBuilder:
    """Split-widest-dimension builds of (N, k) points with a held workspace."""

    def __init__(self, n: int, k: int, device="cuda"):
        import torch
        self.n, self.k = int(n), int(k)
        self.device = torch.device(device)
        nbytes = workspace_size_widest(self.n, self.k)
        if nbytes == 0 and self.n > 1:
            raise ValueError("unsupported size N=%d k=%d" % (self.n, self.k))
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)
        self.workspace_bytes = nbytes

    def _outputs(self, points, perm, tree, dims, want_tree):
        import torch
        _validate_points(points)
        if tuple(points.shape) != (self.n, self.k):
            raise ValueError("points shape %s != (%d, %d)" % (tuple(points.shape), self.n, self.k))
        if perm is None:
            perm = torch.empty(self.n, dtype=torch.int32, device=points.device)
        if tree is None and want_tree:
            tree = torch.empty_like(points)
        if dims is None:
            dims = torch.empty(self.n, dtype=torch.int32, device=points.device)
        return perm, tree, dims

    def build(self, points, perm=None, tree=None, dims=None, want_tree=True, stream=None):
        perm, tree, dims = self._outputs(points, perm, tree, dims, want_tree)
        st = lib().kdt_build_widest(ctypes.c_void_p(points.data_ptr()), self.n, self.k,
                                    ctypes.c_void_p(perm.data_ptr()),
                                    ctypes.c_void_p(tree.data_ptr() if tree is not None else 0),
                                    ctypes.c_void_p(dims.data_ptr()),
                                    ctypes.c_void_p(self.workspace.data_ptr()), self.workspace_bytes,
                                    _stream_handle(points.device, stream))
        _check(st, "kdt_build_widest")
        _used_on(stream, points.device, self.workspace, points, perm, tree, dims)
        return perm, tree, dims

    def build_profiled(self, points, perm, tree=None, dims=None, stream=None):
        perm, tree, dims = self._outputs(points, perm, tree, dims, tree is not None)
        prof = Profile()
        st = lib().kdt_build_widest_profiled(ctypes.c_void_p(points.data_ptr()), self.n, self.k,
                                             ctypes.c_void_p(perm.data_ptr()),
                                             ctypes.c_void_p(tree.data_ptr() if tree is not None else 0),
                                             ctypes.c_void_p(dims.data_ptr()),
                                             ctypes.c_void_p(self.workspace.data_ptr()),
                                             self.workspace_bytes, _stream_handle(points.device, stream),
                                             ctypes.byref(prof))
        _check(st, "kdt_build_widest_profiled")
        return prof.as_dict()


def build_widest(points, want_tree: bool = True, stream=None):
    """Split-widest-dimension tree of `points`: (perm, tree, dims), dims[s]
    (int32) the split dimension of node s."""
    _validate_points(points)
    n, k = points.shape
    return WidestBuilder(n, k, points.device).build(points, want_tree=want_tree, stream=stream)


def build_static(points, want_tree: bool = True, stream=None):
    """The build of `points` through kdt_build_static: the library's static
    scratch array is the workspace, so only the outputs are allocated here.
    Sizes whose workspace exceeds STATIC_SCRATCH_BYTES raise KdtError
    (KDT_ERR_TOO_LARGE). Calls that overlap on one GPU race on that array."""
    import torch
    _validate_points(points)
    n, k = points.shape
    perm = torch.empty(n, dtype=torch.int32, device=points.device)
    tree = torch.empty_like(points) if want_tree else None
    st = lib().kdt_build_static(ctypes.c_void_p(points.data_ptr()), n, k, ctypes.c_void_p(perm.data_ptr()),
                                ctypes.c_void_p(tree.data_ptr() if tree is not None else 0),
                                _stream_handle(points.device, stream))
    _check(st, "kdt_build_static")
    _used_on(stream, points.device, points, perm, tree)
    return perm, tree


def build(points, want_tree: bool = True, stream=None):
    """Build the level-order tree of `points` ((N, k) float32 on a HIP device).

    Returns (perm, tree): perm[s] (int32) is the original index of the point at
    node s; tree[s] = points[perm[s]] (None when want_tree is False)."""
    _validate_points(points)
    n, k = points.shape
    return Builder(n, k, points.device).build(points, want_tree=want_tree, stream=stream)


def knn(tree, perm, queries, K: int, idx=None, d2=None, visits=None, stream=None, budget=None, dims=None,
        wave_stack=None):
    """K nearest neighbours of every query among the points of a built tree.

    tree, perm: the outputs of build() ((N, k) float32 and (N,) int32 on a
    HIP device); queries: (Q, k) float32 on the same device. Returns (idx, d2):
    (Q, K) int32 original indices, nearest first (-1 past N), and their
    (Q, K) float32 squared distances. For a split-widest tree pass its `dims`
    (build_widest's third output). A (Q,) int32 tensor passed as `visits`
    receives the number of tree points each search examined. `budget`
    (diagnostic) sets how many points a first-pass thread examines before
    handing its query to the wave pass; `wave_stack` (diagnostic, 1..2048)
    caps the wave pass's shared stack."""
    import torch
    _validate_points(queries)
    if tree is not None:
        _validate_points(tree)
    n = 0 if tree is None else tree.shape[0]
    k = queries.shape[1]
    if tree is not None and tree.shape[1] != k:
        raise ValueError("tree has k=%d, queries k=%d" % (tree.shape[1], k))
    if perm is not None and (perm.dtype != torch.int32 or perm.numel() != n or not perm.is_contiguous()):
        raise ValueError("perm must be a contiguous int32 tensor of N entries")
    q = queries.shape[0]
    if idx is None:
        idx = torch.empty((q, K), dtype=torch.int32, device=queries.device)
    if d2 is None:
        d2 = torch.empty((q, K), dtype=torch.float32, device=queries.device)
    if dims is not None and (dims.dtype != torch.int32 or dims.numel() != n or not dims.is_contiguous()):
        raise ValueError("dims must be a contiguous int32 tensor of N entries")
    args = [ctypes.c_void_p(tree.data_ptr() if n else 0), ctypes.c_void_p(perm.data_ptr() if n else 0),
            ctypes.c_void_p(dims.data_ptr() if (dims is not None and n) else 0), n, k,
            ctypes.c_void_p(queries.data_ptr()), q, int(K),
            ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(d2.data_ptr()),
            ctypes.c_void_p(visits.data_ptr() if visits is not None else 0)]
    if wave_stack is not None:
        st = lib().kdt_knn_debug(*args, 0xFFFFFFFF if budget is None else int(budget), int(wave_stack),
                                 _stream_handle(queries.device, stream))
    elif budget is None:
        st = lib().kdt_knn(*args, _stream_handle(queries.device, stream))
    else:
        st = lib().kdt_knn_budget(*args, int(budget), _stream_handle(queries.device, stream))
    _check(st, "kdt_knn")
    _used_on(stream, queries.device, tree, perm, dims, queries, idx, d2, visits)
    return idx, d2
