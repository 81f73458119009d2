// Driver for a sanitizer build of the CPU oracle and checker (test
// infrastructure). Reads "N k" and N*k float32 bit patterns (hex) from
// stdin, runs the recursive builder, the ancestor-walking checker and the
// split-widest builder, and prints the results as text. Built with
// AddressSanitizer and UndefinedBehaviorSanitizer (no recovery), so any
// out-of-bounds access or undefined operation ends the process with an error.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

extern "C" {
int kdto_build(const float* pts, int64_t N, int32_t k, int32_t* perm, int nthreads);
int64_t kdto_check(const float* pts, int64_t N, int32_t k, const int32_t* perm);
int kdto_build_widest(const float* pts, int64_t N, int32_t k, int32_t* perm, int32_t* dims, int nthreads);
int64_t kdto_subtree_size(int64_t N, int64_t c);
}

int main() {
    long long n = 0;
    int k = 0;
    if (scanf("%lld %d", &n, &k) != 2 || n < 0 || k < 1) return 2;
    std::vector<float> pts((size_t)n * k);
    for (size_t i = 0; i < pts.size(); ++i) {
        unsigned bits = 0;
        if (scanf("%x", &bits) != 1) return 2;
        memcpy(&pts[i], &bits, sizeof bits);
    }
    std::vector<int32_t> perm((size_t)n), perm_w((size_t)n), dims((size_t)n);
    if (kdto_build(pts.data(), n, k, perm.data(), 2) != 0) return 3;
    const long long bad = (long long)kdto_check(pts.data(), n, k, perm.data());
    if (kdto_build_widest(pts.data(), n, k, perm_w.data(), dims.data(), 2) != 0) return 4;
    // planted mistakes for the checker: a duplicated entry, two children swapped
    long long bad_dup = -1, bad_swap = -1;
    if (n > 2) {
        std::vector<int32_t> dup(perm);
        dup[1] = dup[0];
        bad_dup = (long long)kdto_check(pts.data(), n, k, dup.data());
        std::vector<int32_t> sw(perm);
        const int32_t t = sw[1];
        sw[1] = sw[2];
        sw[2] = t;
        bad_swap = (long long)kdto_check(pts.data(), n, k, sw.data());
    }
    printf("check %lld\nsize %lld\nbad_dup %lld\nbad_swap %lld\n", bad,
           (long long)(n > 1 ? kdto_subtree_size(n, 1) : 0), bad_dup, bad_swap);
    printf("perm");
    for (long long i = 0; i < n; ++i) printf(" %d", perm[(size_t)i]);
    printf("\nwidest");
    for (long long i = 0; i < n; ++i) printf(" %d", perm_w[(size_t)i]);
    printf("\ndims");
    for (long long i = 0; i < n; ++i) printf(" %d", dims[(size_t)i]);
    printf("\n");
    return 0;
}
