"""Pins for the split-widest-dimension oracle (oracle/kdt_widest.cpp); no GPU.

The variant is the one of I. Wald, "GPU-friendly, Parallel, and (Almost-)
In-Place Construction of Left-Balanced k-d Trees" (arXiv 2211.00120),
split-widest-dimension section. The oracle (top-down recursion with explicit
domains) is checked against things other than itself:

* a hand-derived seven-point example (tests/golden/widest_hand_example.txt),
  which also differs from the round-robin tree;
* the page's other formulation, domains clipped bottom-up from each node to
  the root (oracle/widest_check.py), on varied inputs;
* exhaustive search for N <= 7: exactly one arrangement satisfies the
  conditions, and it is the oracle's;
* k = 1: only one dimension, so the tree is the round-robin tree;
* one dominant dimension: while the domain is wide in x every split is in x.

test_planted_mistakes_are_caught recompiles copies of the oracle with one
plausible mistake each; every copy must fail a pin.
"""
import itertools
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import oracle
from oracle import widest_check
from tree_construction_amd import datagen

HERE = os.path.dirname(os.path.abspath(__file__))


def load_hand_example():
    pts, perm, dims = [], None, None
    with open(os.path.join(HERE, "golden", "widest_hand_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, *vals = line.split()
            if tag == "point":
                pts.append([float(v) for v in vals])
            elif tag == "perm":
                perm = [int(v) for v in vals]
            elif tag == "dims":
                dims = [int(v) for v in vals]
    return np.array(pts, dtype=np.float32), perm, dims


def brute_force(pts):
    """Every arrangement that satisfies the variant's conditions (N <= 7):
    dimensions follow from the domains clipped bottom-up, points on the right
    side of every ancestor's plane by (coordinate, index)."""
    n, k = pts.shape
    lo0, hi0 = pts.min(0), pts.max(0)
    found = []
    for perm in itertools.permutations(range(n)):
        dims, ok = [], True
        for s in range(n):
            lo, hi = lo0.copy(), hi0.copy()
            c = s
            while c > 0 and ok:
                a = (c - 1) // 2
                d = dims[a]
                plane = pts[perm[a], d]
                key = (pts[perm[s], d], perm[s])
                if c == 2 * a + 1:
                    ok = key < (plane, perm[a])
                    hi[d] = min(hi[d], plane)
                else:
                    ok = key > (plane, perm[a])
                    lo[d] = max(lo[d], plane)
                c = a
            if not ok:
                break
            ext = (hi - lo).astype(np.float32)
            best = 0
            for d in range(1, k):
                if ext[d] > ext[best]:
                    best = d
            dims.append(best)
        if ok:
            found.append((list(perm), dims))
    return found


# --------------------------------------------------------------- pins

def pin_hand_example(lib):
    pts, perm, dims = load_hand_example()
    p, d = oracle.build_tree_widest(pts, lib=lib)
    return p.tolist() == perm and d.tolist() == dims


def pin_bottom_up_checker(lib):
    cases = [datagen.uniform(3000, 3, 1), datagen.gaussian_mixture(5000, 3, 2), datagen.ties(2000, 3, 3),
             datagen.signed_zeros(700, 2, 4), datagen.all_equal(300, 3), datagen.normal(4097, 5, 5),
             datagen.uniform(1000, 2, 6) * np.array([100.0, 1.0], np.float32),
             datagen.special_values(900, 3, 7)]
    for pts in cases:
        p, d = oracle.build_tree_widest(pts, lib=lib)
        if widest_check.check(pts, p, d) is not None:
            return False
    return True


def pin_brute_force(lib):
    rng = np.random.default_rng(9)
    for n in range(1, 8):
        for trial in range(3):
            k = 2 + trial % 2
            pts = rng.integers(0, 6, (n, k)).astype(np.float32) * np.float32(1 + trial)
            found = brute_force(pts)
            p, d = oracle.build_tree_widest(pts, lib=lib)
            if len(found) != 1 or found[0] != (p.tolist(), d.tolist()):
                return False
    return True


def pin_one_dimension(lib):
    pts = datagen.uniform(1500, 1, 8)
    p, d = oracle.build_tree_widest(pts, lib=lib)
    return np.array_equal(p, oracle.build_tree(pts, lib=lib)) and not d.any()


def pin_dominant_dimension(lib):
    # x spans 1000, y spans 1: the top levels all split x (the domain of a
    # level-l node is about 1000 / 2^l wide in x)
    pts = datagen.uniform(4095, 2, 10) * np.array([1000.0, 1.0], np.float32)
    _, d = oracle.build_tree_widest(pts, lib=lib)
    return not d[:2 ** 8 - 1].any() and d[2 ** 11 - 1:].any()


ALL_PINS = [pin_hand_example, pin_bottom_up_checker, pin_brute_force, pin_one_dimension,
            pin_dominant_dimension]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, oracle_lib):
    assert pin(oracle_lib)


def test_checker_rejects_wrong_trees(oracle_lib):
    pts = datagen.gaussian_mixture(2000, 3, 11)
    p, d = oracle.build_tree_widest(pts)
    assert widest_check.check(pts, p, d) is None
    bad_d = d.copy()
    bad_d[5] = (bad_d[5] + 1) % 3
    assert widest_check.check(pts, p, bad_d) is not None
    bad_p = p.copy()
    bad_p[[3, 4]] = bad_p[[4, 3]]
    assert widest_check.check(pts, bad_p, d) is not None
    # the round-robin tree is not a split-widest tree here
    rr = oracle.build_tree(pts)
    assert widest_check.check(pts, rr, np.arange(2000) * 0 + (np.log2(np.arange(2000) + 1).astype(int) % 3)) is not None


# ------------------------------------------------------ planted mistakes

MUTATIONS = {
    "ties_to_higher_dimension": [("if (extent > best_extent) {", "if (extent >= best_extent) {")],
    "clip_to_the_other_bound": [("left_hi[d] = plane;", "left_hi[d] = lo[d];"),
                                ("right_lo[d] = plane;", "right_lo[d] = hi[d];")],
    "no_clipping": [("left_hi[d] = plane;", ""), ("right_lo[d] = plane;", "")],
    "extent_as_sum": [("float best_extent = hi[0] - lo[0];", "float best_extent = hi[0] + lo[0];"),
                      ("const float extent = hi[d] - lo[d];", "const float extent = hi[d] + lo[d];")],
    "box_from_first_point": [("if (x < lo[d]) lo[d] = x;", ""), ("if (hi[d] < x) hi[d] = x;", "")],
    "narrowest_dimension": [("if (extent > best_extent) {", "if (extent < best_extent) {")],
}


def _run_pins_in_child(lib_path):
    code = ("import sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
            "import oracle, test_widest_oracle as t\n"
            "lib = oracle.load_lib(%r)\n"
            "bad = [p.__name__ for p in t.ALL_PINS if not p(lib)]\n"
            "print('FAILED_PINS', bad)\n"
            "sys.exit(3 if bad else 0)\n" % (os.path.dirname(HERE), HERE, lib_path))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout + r.stderr


def test_unmutated_oracle_passes_in_child():
    rc, out = _run_pins_in_child(oracle.load_lib() and oracle.LIB_PATH)
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name, tmp_path):
    src_dir = os.path.dirname(oracle.__file__)
    for f in oracle._SOURCES:
        shutil.copy(os.path.join(src_dir, f), tmp_path / f)
    path = tmp_path / "kdt_widest.cpp"
    text = path.read_text()
    for old, new in MUTATIONS[name]:
        assert old in text, "mutation anchor missing: %r" % old
        text = text.replace(old, new, 1)
    path.write_text(text)
    lib_path = oracle.compile_lib(str(tmp_path), str(tmp_path / "libmut.so"))
    rc, out = _run_pins_in_child(lib_path)
    assert rc != 0, "mutation %s slipped past every pin:\n%s" % (name, out)
