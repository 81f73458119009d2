/*
 * kdt.h -- C ABI of the MI355X (gfx950) left-balanced k-d tree builder.
 *
 * What it builds: the left-balanced, complete k-d tree over N points of
 * dimension k, stored in level order with no pointers (node s has children
 * 2s+1 and 2s+2; node s on level l = floor(log2(s+1)) splits in dimension
 * l mod k), as defined in I. Wald, "GPU-friendly, Parallel, and
 * (Almost-)In-Place Construction of Left-Balanced k-d Trees" (arXiv
 * 2211.00120): the problem statement (k-d condition plus balancing
 * condition), the indexing paragraph (level-order ids, lChild/rChild, level,
 * numLevels, F(l)) and the assumptions paragraph (dimension l mod k).
 * Coordinates are ordered by IEEE '<' (so -0.0 == +0.0) with the original
 * point index as the tie-break, which makes the tree unique.
 *
 * How: the paper's tag-based "trickle-down" construction. Every point
 * carries a tag, the id of its ancestor on the current level (tag
 * paragraph); each round sorts all points by (tag, coordinate l mod k,
 * original index) and refines every tag from the closed-form subtree sizes
 * and segment starts (sort-order and sb/ss paragraphs). On the GPU each
 * split dimension keeps an array of point records in that round order,
 * built by a stable LSD radix sort of (coordinate, index) when the
 * dimension is first used. A tag update is a comparison with the pivot of
 * the point's node, so a round re-sorts its dimension's array by the new
 * tags with one stable radix pass whose digit is the point's path down the
 * pivots of the levels since that array was last sorted; the pivots of the
 * round then sit at closed-form positions. A round whose array is not
 * needed in that order again only locates its pivots (counts, then the
 * tiles that hold them). Subtrees of at most 4096 points finish their
 * remaining rounds inside one workgroup's LDS.
 *
 * Conventions for every entry point:
 *   - All pointers marked "device" are HIP device pointers on the current
 *     device. The caller owns every buffer; the library allocates nothing,
 *     keeps no global state and is re-entrant: calls on different streams
 *     with different workspaces may run concurrently. The one exception is
 *     kdt_build_static, whose workspace is a static device array per GPU.
 *   - All work is enqueued on `stream` (0 = the null stream) and the call
 *     returns before it finishes; synchronise the stream before reading
 *     outputs. Argument errors are detected before anything is enqueued.
 *   - Limits: 0 <= N <= 2^31 - 1, 1 <= k <= 65535. NaN coordinates are
 *     outside the definition: the build stays in bounds and returns some
 *     permutation, but which one is unspecified.
 */
#ifndef KDT_H
#define KDT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t (redeclaring an identical typedef is legal). */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
    KDT_OK = 0,
    KDT_ERR_INVALID_ARG = 1, /* bad N or k, NULL pointer, overlapping buffers */
    KDT_ERR_WORKSPACE = 2,   /* workspace NULL or smaller than kdt_workspace_size() */
    KDT_ERR_HIP = 3,         /* a kernel launch failed (hipGetLastError) */
    KDT_ERR_TOO_LARGE = 4    /* kdt_build_static: N, k need more than its scratch array */
} kdt_status;

/* Bytes of device workspace kdt_build() needs for N points of dimension k.
 * Pure host arithmetic, no HIP call. Returns 0 when N or k is out of range
 * (and for N <= 1, which needs none). */
size_t kdt_workspace_size(int64_t N, int32_t k);

/* Build the tree.
 *   points    device, N*k float32, row-major: point i's coordinate d is
 *             points[i*k + d]. Read only.
 *   perm_out  device, N int32: perm_out[s] = original index of the point at
 *             level-order node s.
 *   tree_out  device, N*k float32 or NULL: tree_out[s*k + d] =
 *             points[perm_out[s]*k + d], a bit copy (-0.0 stays -0.0).
 *   workspace device, at least kdt_workspace_size(N, k) bytes, 256-byte
 *             aligned; its contents on entry do not matter and are
 *             clobbered. May be NULL when N <= 1.
 * perm_out and tree_out must not overlap points, each other or the
 * workspace. On any error the outputs are unspecified. */
kdt_status kdt_build(const float* points, int64_t N, int32_t k,
                     int32_t* perm_out, float* tree_out,
                     void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Allocation-free build, for callers that cannot call hipMalloc (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Identical to kdt_build, except that the workspace is a file-scope device
 * array of KDT_STATIC_SCRATCH_BYTES bytes inside the library (one per GPU,
 * held until the process ends; its device address is looked up once per
 * device on the first call made with that device current). The caller still
 * passes the points and the outputs, as for kdt_build.
 *   Returns KDT_ERR_TOO_LARGE, before anything is enqueued, when
 *   kdt_workspace_size(N, k) > KDT_STATIC_SCRATCH_BYTES (for k = 3 that is
 *   N above about 666,000 points).
 *   Every call on one GPU shares that GPU's array and it keeps the last
 *   call's contents (the build needs no zeroed workspace). Calls that overlap
 *   on one GPU (on different streams, or from several threads without
 *   ordering) race on it and give unspecified outputs: serialise them.
 * Other arguments, the stream rule and the errors are those of kdt_build. */
#define KDT_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
kdt_status kdt_build_static(const float* points, int64_t N, int32_t k,
                            int32_t* perm_out, float* tree_out, hipStream_t stream);

/* Diagnostic: run only the first `rounds` sort+update rounds (0 <= rounds
 * <= numLevels(N) - 1) over the whole point set and copy every point's tag
 * to tags_out (device, N uint32, indexed by original point index). After r
 * rounds the tag of a point is its final node's ancestor on level r (or the
 * node itself when it sits on a level < r), as the paper's tag paragraph
 * states; here it is read off the pivots those rounds fixed. The workspace
 * must hold kdt_debug_workspace_size(N, k, rounds) bytes; otherwise the
 * same error rules as kdt_build. */
kdt_status kdt_debug_tags(const float* points, int64_t N, int32_t k, int32_t rounds,
                          uint32_t* tags_out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Bytes of workspace kdt_debug_tags() needs (pure host arithmetic; 0 when
 * the arguments are out of range or no workspace is needed). */
size_t kdt_debug_workspace_size(int64_t N, int32_t k, int32_t rounds);

/* Per-kernel-kind timing of one build, for benchmarking. */
#define KDT_PROFILE_MAX_KINDS 32
#define KDT_PROFILE_NAME_LEN 48
typedef struct {
    int32_t kinds;                        /* entries filled below */
    char name[KDT_PROFILE_MAX_KINDS][KDT_PROFILE_NAME_LEN]; /* kernel as the profiler
                                             prints it, NUL-terminated, e.g.
                                             "k_part_scatter<4>" */
    int64_t launches[KDT_PROFILE_MAX_KINDS];
    double ms[KDT_PROFILE_MAX_KINDS];     /* summed GPU duration (HIP events) */
    double bytes[KDT_PROFILE_MAX_KINDS];  /* summed algorithmic bytes: each array
                                             a kernel must read or write, once */
} kdt_profile;

/* kdt_build with a HIP event pair recorded on `stream` around every kernel
 * launch. Synchronises the stream before returning, then fills *profile
 * (durations include only GPU time between each pair). Same arguments and
 * errors as kdt_build, plus KDT_ERR_INVALID_ARG for profile == NULL. */
kdt_status kdt_build_profiled(const float* points, int64_t N, int32_t k,
                              int32_t* perm_out, float* tree_out,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream, kdt_profile* profile);

/* Host copies of the closed forms the kernels evaluate (no HIP call), for
 * tests: the size of level-order subtree s in a complete tree of N nodes
 * (0 if s >= N), and the first sorted position of subtree s's points after
 * the round that fixes level l (s on level l, 0 <= l <= numLevels(N) - 1;
 * returns -1 when s is not on level l or the arguments are out of range). */
int64_t kdt_closed_subtree_size(int64_t N, int64_t s);
int64_t kdt_closed_segment_begin(int64_t N, int64_t s, int32_t l);

/* Host copies of the closed forms the per-round re-sort evaluates (no HIP
 * call), for tests. A point is live on level l when it is not yet a node
 * above l; in round l's order the live points of the subtree of the j-th
 * node on level l start at live position kdt_closed_segment_begin(N,
 * F(l)+j, l) - F(l).
 *   kdt_closed_live_segment: the j whose subtree holds live position p on
 *     level l (-1 when l or p is out of range).
 *   kdt_closed_bin_prefix: the number of points in the subtrees of the
 *     first j0 nodes on level l1 - delta whose ancestor on level l1 is the
 *     b-th level-l1 node below their level-(l1 - delta) one, i.e. the sum
 *     of |S| over the level-l1 nodes with in-level index j*2^delta + b,
 *     j < j0 (0 <= delta <= min(l1, 8), 0 <= j0 <= 2^(l1-delta),
 *     0 <= b < 2^delta; -1 otherwise). */
int64_t kdt_closed_live_segment(int64_t N, int32_t l, int64_t p);
int64_t kdt_closed_bin_prefix(int64_t N, int32_t l1, int32_t delta, int64_t j0, int64_t b);

/* Host copy of the coordinate key every kernel compares (no HIP call), for
 * tests: keys_out[i] = key of the float32 bit pattern bits[i], an unsigned
 * 32-bit value whose order is IEEE '<' on the floats, with -0.0 and +0.0
 * mapped to one key (the problem statement's k-d condition compares values,
 * and the tie-break is the index). NaN patterns get some key (outside the
 * definition). n < 0 or NULL pointers with n > 0: nothing is written. */
void kdt_closed_float_keys(const uint32_t* bits, int64_t n, uint32_t* keys_out);

/* Split-widest-dimension variant ([W], split-widest-dimension section).
 * The same left-balanced complete level-order tree, except that node s
 * splits along the dimension in which its domain is widest: the root's
 * domain is the bounding box of all points (per-dimension minimum and
 * maximum); a child's domain is its parent's, bounded at the parent's point
 * in the parent's dimension (upper bound on the left, lower bound on the
 * right); "widest" compares float32 extents hi - lo and takes the lowest
 * dimension on ties. The point at s is the element of rank |S(2s+1)| of
 * its subtree's points by (coordinate in s's dimension, original index).
 *   dims_out  device, N int32 or NULL: dims_out[s] = split dimension of
 *             node s (every node, leaves included).
 * Other arguments, ownership and errors as kdt_build; the workspace is
 * kdt_workspace_size_widest(N, k) bytes. Subtrees of at most 4096 points
 * finish in LDS. Above them, for k <= 3 each dimension's array finds its
 * own nodes' pivots on every level, so a build costs more than kdt_build's;
 * for k > 3 every level sorts all points by their node's own dimension. */
size_t kdt_workspace_size_widest(int64_t N, int32_t k);
kdt_status kdt_build_widest(const float* points, int64_t N, int32_t k,
                            int32_t* perm_out, float* tree_out, int32_t* dims_out,
                            void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* kdt_build_widest with per-kernel timing, as kdt_build_profiled. */
kdt_status kdt_build_widest_profiled(const float* points, int64_t N, int32_t k,
                                     int32_t* perm_out, float* tree_out, int32_t* dims_out,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream, kdt_profile* profile);

/* Duplicate removal, the optional pre-pass of J. Robinson's KdTreeGPU
 * wiki (duplicate-removal section): tuples equal in every coordinate
 * (IEEE '==', so -0.0 equals +0.0) collapse to one. Of each group of equal
 * tuples the one with the smallest original index is kept. The GPU sorts
 * (32-bit tuple hash, index) pairs, so equal tuples meet in index order,
 * and compares coordinates exactly inside runs of equal hashes: distinct
 * tuples that share a hash cost time, never a wrong answer.
 *   points     device, N*k float32, row-major. Read only.
 *   keep_out   device, N int32: its first *count_out entries are the kept
 *              indices, ascending; the rest are unspecified.
 *   count_out  device, one int64: the number of distinct tuples.
 * Workspace: kdt_unique_workspace_size(N, k) bytes, 256-byte aligned.
 * Ownership, streams and errors as kdt_build (NULL count_out is
 * KDT_ERR_INVALID_ARG). NaN coordinates are outside the definition. */
size_t kdt_unique_workspace_size(int64_t N, int32_t k);
kdt_status kdt_unique(const float* points, int64_t N, int32_t k,
                      int32_t* keep_out, int64_t* count_out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* kdt_unique with per-kernel timing, as kdt_build_profiled. */
kdt_status kdt_unique_profiled(const float* points, int64_t N, int32_t k,
                               int32_t* keep_out, int64_t* count_out,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream, kdt_profile* profile);

/* K nearest neighbours of each query point among the N points of a tree
 * built by kdt_build or kdt_build_widest, exactly as a brute-force search
 * ranks them. The search is the two-phase descent and backtrack of
 * F. Gieseke et al., "Bigger Buffer k-d Trees on Multi-Many-Core Systems"
 * (arXiv 1512.02831), section 2.3, over the left-balanced level-order tree.
 * Distances are float32 squared Euclidean distances, summed in dimension
 * order with separately rounded products and sums; neighbours are ordered
 * by (squared distance, original index).
 *   tree      device, N*k float32: the tree_out of kdt_build (level order).
 *   perm      device, N int32: the perm_out of the same build.
 *   dims      device, N int32 or NULL: the dims_out of kdt_build_widest
 *             (each node's split dimension); NULL for a kdt_build tree
 *             (node s splits dimension level(s) mod k).
 *   queries   device, Q*k float32, row-major. Read only.
 *   K         neighbours per query, 1 <= K <= 32.
 *   idx_out   device, Q*K int32: row q holds the original indices of query
 *             q's K nearest points, nearest first; -1 where N < K.
 *   d2_out    device, Q*K float32 or NULL: the matching squared distances
 *             (+inf where N < K).
 *   visits_out device, Q uint32 or NULL: the number of tree points the
 *             search of each query examined (N when K >= N; a query that
 *             the wave pass finishes counts both passes' points).
 * Coordinates of points and queries must be finite. 0 <= N, Q <= 2^31 - 1;
 * 1 <= k <= 65535. The outputs must not overlap the inputs or each other.
 * Allocates nothing; enqueued on `stream` (two kernels: one thread per
 * query, then one wave per query whose search outgrew the first pass);
 * argument errors (KDT_ERR_INVALID_ARG) are detected before anything is
 * enqueued. */
kdt_status kdt_knn(const float* tree, const int32_t* perm, const int32_t* dims,
                   int64_t N, int32_t k, const float* queries, int64_t Q, int32_t K,
                   int32_t* idx_out, float* d2_out, uint32_t* visits_out,
                   hipStream_t stream);

/* Diagnostic: kdt_knn with the first pass's budget given. A first-pass
 * thread examines at most `budget` tree points before handing its query to
 * the wave pass (kdt_knn uses 32 K, clamped to [128, 512]); 0 hands every
 * query over. The results do not depend on the budget. Same arguments and
 * errors as kdt_knn. */
kdt_status kdt_knn_budget(const float* tree, const int32_t* perm, const int32_t* dims,
                          int64_t N, int32_t k, const float* queries, int64_t Q, int32_t K,
                          int32_t* idx_out, float* d2_out, uint32_t* visits_out,
                          uint32_t budget, hipStream_t stream);

/* Diagnostic: kdt_knn_budget with the wave pass's shared stack capped at
 * `wave_stack` entries (1 <= wave_stack <= 2048; kdt_knn uses 2048; else
 * KDT_ERR_INVALID_ARG). When a step's far sides do not fit, each lane walks
 * its own by parent links, so a small cap exercises that path. budget =
 * 0xFFFFFFFF selects kdt_knn's own budget. The results depend on neither.
 * Same arguments and errors as kdt_knn otherwise. */
kdt_status kdt_knn_debug(const float* tree, const int32_t* perm, const int32_t* dims,
                         int64_t N, int32_t k, const float* queries, int64_t Q, int32_t K,
                         int32_t* idx_out, float* d2_out, uint32_t* visits_out,
                         uint32_t budget, uint32_t wave_stack, hipStream_t stream);

/* Static description of a status code. */
const char* kdt_status_string(kdt_status status);

#ifdef __cplusplus
}
#endif

#endif /* KDT_H */
