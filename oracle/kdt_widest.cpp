/*
 * CPU oracle for the split-widest-dimension variant of the left-balanced,
 * complete, level-order k-d tree.
 *
 * TEST INFRASTRUCTURE (like kdt_oracle.cpp): only the test suite, smoke()
 * and the benchmark's CPU-baseline leg load it; it shares nothing with the
 * HIP library.
 *
 * Source: I. Wald, "GPU-friendly, Parallel, and (Almost-)In-Place
 * Construction of Left-Balanced k-d Trees" (arXiv 2211.00120), section on
 * the split-widest-dimension variant, cited as [W]. There the recursive
 * builder is described first: compute the bounding box of all points (the
 * domain of the root); at each subtree, split along the dimension in which
 * the subtree's domain is widest; the children's domains are the parent's,
 * cut by the parent's splitting plane; recurse. This file is that builder.
 *
 * Readings fixed here (the page leaves them open):
 *   - the root domain is the per-dimension minimum and maximum of all
 *     points' coordinates;
 *   - "widest" compares the float32 extents hi[d] - lo[d] (one rounded
 *     subtraction each) with '>', scanning d = 0 .. k-1, so the lowest
 *     dimension wins ties;
 *   - a node's plane is its point's coordinate in its split dimension: the
 *     left child's domain takes it as its upper bound there, the right
 *     child's as its lower bound;
 *   - everything else is the round-robin tree's definition: the point at s
 *     is the element of rank |S(2s+1)| of its subtree's points ordered by
 *     (coordinate in s's dimension, original index), smaller ones to the
 *     left. Every node, leaves included, gets a split dimension.
 * NaN coordinates are outside the definition.
 */
#include <algorithm>
#include <cstdint>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

/* |S(c)| in a complete level-order tree of N nodes: count c's descendants
 * level by level through the children ids ([W], indexing paragraph). */
int64_t count_subtree(int64_t N, int64_t c) {
    int64_t count = 0, lo = c, hi = c;
    while (lo < N) {
        count += (hi < N ? hi : N - 1) - lo + 1;
        lo = 2 * lo + 1;
        hi = 2 * hi + 2;
    }
    return count;
}

/* Dimension of the widest extent of the domain [lo, hi]. */
int widest(const std::vector<float>& lo, const std::vector<float>& hi) {
    int best = 0;
    float best_extent = hi[0] - lo[0];
    for (size_t d = 1; d < lo.size(); ++d) {
        const float extent = hi[d] - lo[d];
        if (extent > best_extent) {
            best = (int)d;
            best_extent = extent;
        }
    }
    return best;
}

struct Ctx {
    const float* pts;
    int64_t N, k;
    int32_t* perm;
    int32_t* dims;
    int64_t task_cutoff;
};

struct ByCoordinate {
    const float* pts;
    int64_t k;
    int d;
    bool operator()(int32_t a, int32_t b) const {
        const float xa = pts[(int64_t)a * k + d], xb = pts[(int64_t)b * k + d];
        if (xa < xb) return true;
        if (xb < xa) return false;
        return a < b;
    }
};

void build(const Ctx& c, int32_t* idx, int64_t n, int64_t s, std::vector<float> lo,
           std::vector<float> hi) {
    if (n == 0) return;
    const int d = widest(lo, hi);
    c.dims[s] = d;
    std::sort(idx, idx + n, ByCoordinate{c.pts, c.k, d});
    const int64_t m = count_subtree(c.N, 2 * s + 1);
    c.perm[s] = idx[m];
    const float plane = c.pts[(int64_t)idx[m] * c.k + d];
    std::vector<float> left_hi = hi, right_lo = lo;
    left_hi[d] = plane;
    right_lo[d] = plane;
    int32_t* left = idx;
    int32_t* right = idx + m + 1;
    const int64_t nl = m, nr = n - m - 1;
    if (n > c.task_cutoff) {
#pragma omp task default(none) firstprivate(left, nl, s, lo, left_hi) shared(c)
        build(c, left, nl, 2 * s + 1, lo, left_hi);
#pragma omp task default(none) firstprivate(right, nr, s, right_lo, hi) shared(c)
        build(c, right, nr, 2 * s + 2, right_lo, hi);
#pragma omp taskwait
    } else {
        build(c, left, nl, 2 * s + 1, lo, left_hi);
        build(c, right, nr, 2 * s + 2, right_lo, hi);
    }
}

}  // namespace

extern "C" {

/* Build the split-widest tree: perm[s] = original index at node s, dims[s]
 * = split dimension of node s (both N entries). Returns 0, or -1 on bad
 * arguments. nthreads <= 0 uses the OpenMP default. */
int kdto_build_widest(const float* pts, int64_t N, int32_t k, int32_t* perm, int32_t* dims,
                      int nthreads) {
    if (N < 0 || k < 1 || N > INT32_MAX) return -1;
    if (N == 0) return 0;
    if (!pts || !perm || !dims) return -1;
    std::vector<float> lo(pts, pts + k), hi(pts, pts + k);
    for (int64_t i = 1; i < N; ++i)
        for (int d = 0; d < k; ++d) {
            const float x = pts[i * k + d];
            if (x < lo[d]) lo[d] = x;
            if (hi[d] < x) hi[d] = x;
        }
    std::vector<int32_t> idx((size_t)N);
    for (int64_t i = 0; i < N; ++i) idx[(size_t)i] = (int32_t)i;
    Ctx c{pts, N, (int64_t)k, perm, dims, (int64_t)1 << 15};
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel default(none) shared(c, idx, N, lo, hi)
#pragma omp single
#endif
    build(c, idx.data(), N, 0, lo, hi);
    return 0;
}

}  /* extern "C" */
