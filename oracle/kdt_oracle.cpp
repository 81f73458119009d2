/*
 * CPU oracle for the left-balanced, complete, level-order k-d tree.
 *
 * TEST INFRASTRUCTURE. This is the slow, plainly-correct definition that the
 * GPU build is checked against. Only the test suite, the package's smoke()
 * check and the benchmark's CPU-baseline leg may load it. It shares no code,
 * header, table or helper with the HIP library, and includes nothing from it.
 *
 * Source: I. Wald, "GPU-friendly, Parallel, and (Almost-)In-Place
 * Construction of Left-Balanced k-d Trees" (arXiv 2211.00120), cited below
 * as [W] with the paragraph that states each fact.
 *
 * What is computed. For N points of dimension k (row-major, point i's
 * coordinate d at pts[i*k+d]) the output perm[] maps each level-order node
 * id to the original index of the point stored there. Node s has children
 * 2s+1 and 2s+2 ([W], indexing paragraph: lChild/rChild), so the tree shape
 * is fixed by N alone. Every node s on level l splits in dimension l mod k
 * ([W], assumptions paragraph: round-robin dimension). The point at s is the
 * element of rank |S(2s+1)| of its subtree's points in the order "coordinate
 * d, then original index"; the smaller ones form the left subtree, the
 * larger ones the right subtree. That satisfies the k-d condition (left <=
 * node <= right in the node's dimension) and the balancing condition (the
 * left-balanced complete shape fixes every subtree's size), the two
 * conditions of [W]'s problem statement. The index tie-break makes the
 * order strict, so the tree is unique.
 *
 * Algorithm: the "usual" recursive builder that [W] describes before its own
 * method: sort the array, split it at the position that keeps the tree
 * balanced, recurse on both halves. std::sort is the sort. Float comparison
 * is IEEE '<' (so -0.0 equals +0.0 and the index decides); NaN inputs are
 * outside the definition. Build without -ffast-math so denormals compare
 * exactly.
 *
 * Parity: pinned by the brute-force, closed-form and special-case tests in
 * tests/test_oracle_pins.py (the page's own intermediate tables and its
 * results table are not part of the extracted text).
 */
#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

/* Number of nodes in the level-order subtree rooted at c of a complete tree
 * with N nodes ([W], indexing paragraph: sub-tree S(i)). The descendants of c
 * t levels down are the contiguous ids [lo, hi] obtained by applying
 * lChild to lo and rChild to hi t times; count them while they exist. */
int64_t subtree_size(int64_t N, int64_t c) {
    int64_t count = 0;
    int64_t lo = c, hi = c;
    while (lo < N) {
        int64_t last = hi < N ? hi : N - 1;
        count += last - lo + 1;
        lo = 2 * lo + 1;
        hi = 2 * hi + 2;
    }
    return count;
}

struct Ctx {
    const float* pts;
    int64_t N;
    int64_t k;
    int32_t* perm;
    int64_t task_cutoff;
};

/* Order "coordinate d first, original index second" (strict total order). */
struct Less {
    const float* pts;
    int64_t k;
    int d;
    bool operator()(int32_t a, int32_t b) const {
        float xa = pts[(int64_t)a * k + d];
        float xb = pts[(int64_t)b * k + d];
        if (xa < xb) return true;
        if (xb < xa) return false;
        return a < b;
    }
};

/* Build subtree s (on level l) from the n original indices in idx[]. */
void build_subtree(const Ctx& c, int32_t* idx, int64_t n, int64_t s, int l) {
    if (n == 0) return;                       /* s >= N: no such node */
    int d = (int)(l % c.k);                   /* round-robin split dimension */
    std::sort(idx, idx + n, Less{c.pts, c.k, d});
    int64_t m = subtree_size(c.N, 2 * s + 1); /* size of the left subtree */
    c.perm[s] = idx[m];
    int32_t* left = idx;
    int32_t* right = idx + m + 1;
    int64_t nl = m, nr = n - m - 1;
    if (n > c.task_cutoff) {
#pragma omp task default(none) firstprivate(left, nl, s, l) shared(c)
        build_subtree(c, left, nl, 2 * s + 1, l + 1);
#pragma omp task default(none) firstprivate(right, nr, s, l) shared(c)
        build_subtree(c, right, nr, 2 * s + 2, l + 1);
#pragma omp taskwait
    } else {
        build_subtree(c, left, nl, 2 * s + 1, l + 1);
        build_subtree(c, right, nr, 2 * s + 2, l + 1);
    }
}

}  // namespace

extern "C" {

/* Size of the subtree rooted at node c in a complete level-order tree of N
 * nodes (0 when c >= N). */
int64_t kdto_subtree_size(int64_t N, int64_t c) {
    if (N <= 0 || c < 0) return 0;
    return subtree_size(N, c);
}

/* Build the tree. pts: N*k floats, row-major. perm: N int32 outputs.
 * nthreads <= 0 uses the OpenMP default. Returns 0, or -1 on bad arguments. */
int kdto_build(const float* pts, int64_t N, int32_t k, int32_t* perm, int nthreads) {
    if (N < 0 || k < 1 || N > INT32_MAX) return -1;
    if (N == 0) return 0;
    if (!pts || !perm) return -1;
    std::vector<int32_t> idx((size_t)N);
    for (int64_t i = 0; i < N; ++i) idx[(size_t)i] = (int32_t)i;
    Ctx c{pts, N, (int64_t)k, perm, (int64_t)1 << 15};
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel default(none) shared(c, idx, N)
#pragma omp single
#endif
    build_subtree(c, idx.data(), N, 0, 0);
    return 0;
}

/* Number of threads an OpenMP parallel region would use (1 without OpenMP). */
int kdto_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

}  /* extern "C" */
