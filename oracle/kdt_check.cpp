/*
 * Checker for a level-order k-d tree permutation.
 *
 * TEST INFRASTRUCTURE. Like the oracle beside it, only the test suite,
 * smoke() and the benchmark's CPU-baseline leg may load it, and it shares no
 * code with the HIP library. It also shares no code with kdt_oracle.cpp: it
 * does not build anything, it walks every node's ancestors and tests the
 * definition directly.
 *
 * Source: I. Wald, "GPU-friendly, Parallel, and (Almost-)In-Place
 * Construction of Left-Balanced k-d Trees" (arXiv 2211.00120) [W].
 *
 * A permutation perm (level-order node id -> original point index) is the
 * tree iff
 *   (1) it is a permutation of 0..N-1, and
 *   (2) for every node n and every proper ancestor a of n, with
 *       d = level(a) mod k and "<" the order (coordinate d, then index):
 *       point(n) < point(a) when n lies in a's left subtree, and
 *       point(a) < point(n) when n lies in a's right subtree.
 * (2) is [W]'s k-d condition with the index tie-break; the subtree sizes
 * of [W]'s balancing condition hold by construction because node ids
 * 0..N-1 of a level-order array always form the complete left-balanced
 * shape. With the strict order the tree satisfying (1)+(2) is unique (the
 * node's rank inside its subtree is forced to equal its left-subtree size),
 * so passing this check is equivalent to equality with the oracle.
 * level(i) = floor(log2(i+1)); parent(i) = (i-1)/2 ([W], indexing paragraph).
 */
#include <cstddef>
#include <cstdint>
#include <vector>

namespace {

int level_of(int64_t i) {
    int l = 0;
    for (uint64_t v = (uint64_t)i + 1; v > 1; v >>= 1) ++l;
    return l;
}

bool less_at(const float* pts, int64_t k, int d, int32_t a, int32_t b) {
    float xa = pts[(int64_t)a * k + d];
    float xb = pts[(int64_t)b * k + d];
    if (xa < xb) return true;
    if (xb < xa) return false;
    return a < b;
}

}  // namespace

extern "C" {

/* Returns -1 if perm is the tree. Otherwise returns the first offending node
 * found (for a non-permutation: N + the first duplicated/out-of-range slot).
 * Runs in O(N log N) time; parallel over nodes with OpenMP. */
int64_t kdto_check(const float* pts, int64_t N, int32_t k, const int32_t* perm) {
    if (N <= 0) return -1;
    std::vector<unsigned char> seen((size_t)N, 0);
    for (int64_t n = 0; n < N; ++n) {
        int32_t p = perm[n];
        if (p < 0 || p >= N || seen[(size_t)p]) return N + n;
        seen[(size_t)p] = 1;
    }
    int64_t bad = N;  /* smallest failing node, N if none */
#pragma omp parallel for schedule(static) reduction(min : bad)
    for (int64_t n = 1; n < N; ++n) {
        int32_t pn = perm[n];
        int64_t child = n;
        while (child > 0) {
            int64_t a = (child - 1) / 2;
            int d = level_of(a) % k;
            bool in_left = (child == 2 * a + 1);
            int32_t pa = perm[a];
            bool ok = in_left ? less_at(pts, k, d, pn, pa) : less_at(pts, k, d, pa, pn);
            if (!ok) {
                if (n < bad) bad = n;
                break;
            }
            child = a;
        }
    }
    return bad == N ? -1 : bad;
}

}  /* extern "C" */
