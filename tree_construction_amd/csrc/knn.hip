// knn.hip -- K nearest neighbours over the left-balanced level-order tree
// that kdt_build writes, on MI355X (gfx950).
//
// The search is the two-phase one of F. Gieseke et al., "Bigger Buffer k-d
// Trees on Multi-Many-Core Systems" (arXiv 1512.02831), section 2.3: go down
// the tree to the cell of the query, then back up, and on the way check the
// other side of every splitting plane that lies closer to the query than the
// current K-th neighbour. Here every node is a point (I. Wald's left-balanced
// tree: node s has children 2s+1, 2s+2 and splits dimension level(s) mod k),
// so each node visited on the way down is also a candidate. The way back up
// follows the implicit parent links (s-1)/2 instead of a stack: a thread
// remembers only the node it came from.
//
// Most searches examine a few hundred points, but a few (queries in sparse
// regions next to dense clusters) examine tens of thousands, and one thread
// per query would leave the whole pass waiting for them. So a thread gives up
// after a budget of points and marks the query; a second pass then runs each
// marked query on a whole wave: the lanes pop subtrees from a shared stack in
// LDS, each with a lower bound on its squared distance, and insert their
// candidates into one K-best list spread over the wave's lanes, so every
// lane prunes with the query's own K-th distance so far. The K-th distance
// the first pass had reached when it gave up bounds the answer's from the
// start, and is handed over in the query's mark.
//
// Exactness. Distances are float32 squared distances summed in dimension
// order with separately rounded products and sums, and neighbours are ranked
// by (squared distance, original index), as the brute-force reference does.
// The far side of a plane is skipped only when the squared plane distance is
// strictly larger than the K-th squared distance: every point there differs
// from the query by at least the plane distance in that dimension, rounding
// is monotone, and a sum of non-negative rounded terms is at least each term,
// so no skipped point could rank within the K (ties included). The result is
// therefore identical to brute force, not an approximation.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kdt.h"

namespace {

typedef uint32_t u32;
typedef uint64_t u64;
typedef int64_t i64;

constexpr int kKnnBlock = 256;
constexpr int kPathRegs = 10;  // split offsets of the deepest path nodes a search thread keeps
constexpr int kKnnMaxK = 32;       // neighbours per query at most
// Points one first-pass thread examines before handing its query over:
// 32 K within [128, 512], about the 99th percentile of a typical search (the
// work grows with K). The wave pass is cheap enough that handing over early
// pays, down to a point: on a 16M-point tree (1M queries) this was the best
// budget for K = 1, 8 and 32 (128, 256, 512), where half or twice it cost
// 10-70 % more.
inline u32 default_budget(int K) {
    const u32 b = 32u * (u32)K;
    return b < 128u ? 128u : (b > 512u ? 512u : b);
}
constexpr int kWaveStack = 2048;   // shared stack entries of a wave's search
// First output index of a query handed to a wave: kHandedOver when the first
// pass found fewer than K points, else kHandedOver - 1 - b for the float
// bits b of its K-th squared distance (a finite or infinite square has
// b <= 0x7f800000, so the mark stays within int32).
constexpr int32_t kHandedOver = -2;
constexpr u32 kInfBits = 0x7f800000u;

struct KnnArgs {
    const float* tree;   // N x k, level order
    const int32_t* perm; // N: original index of each node's point
    const int32_t* dims; // N split dimensions (split-widest trees) or nullptr: level mod k
    i64 n;
    int k;
    const float* queries;  // Q x k
    i64 q;
    int K;
    int32_t* idx_out;    // Q x K
    float* d2_out;       // Q x K or nullptr
    uint32_t* visits_out;  // Q or nullptr: nodes examined per query
    u32 budget;          // points a first-pass thread examines before handing over
    u32 wave_stack;      // entries of the wave pass's LDS stack in use (<= kWaveStack)
};

// The query's coordinates: kDims > 0 keeps them in registers (k == kDims);
// kDims == 0 reads them from memory (any k).
template <int kDims>
struct Query {
    float c[kDims > 0 ? kDims : 1];
    const float* row;

    __device__ __forceinline__ void load(const float* queries, u64 qi, int k) {
        row = queries + qi * (u64)k;
        if constexpr (kDims > 0) {
#pragma unroll
            for (int d = 0; d < kDims; ++d) c[d] = row[d];
        }
    }
    // coordinate d (uniform or not), picked with bit masks so that the
    // compiler cannot turn the choice into an indexed (scratch) array
    __device__ __forceinline__ float at(int d) const {
        if constexpr (kDims == 0) {
            return row[d];
        } else {
            u32 v = 0;
#pragma unroll
            for (int i = 0; i < kDims; ++i) v |= __float_as_uint(c[i]) & (d == i ? ~0u : 0u);
            return __uint_as_float(v);
        }
    }
};

// A node's point as the search needs it: the coordinate in its split
// dimension and (for the distance) the row. With k <= 4 the whole row is
// loaded together with the node's dimension, so neither load waits for the
// other; picking the split coordinate is then register work.
template <int kDims>
struct NodeRow {
    float p[kDims > 0 ? kDims : 1];
    const float* row;

    __device__ __forceinline__ void load(const float* tree, u32 node, int k) {
        row = tree + (u64)node * (u64)k;
        if constexpr (kDims > 0) {
#pragma unroll
            for (int d = 0; d < kDims; ++d) p[d] = row[d];
        }
    }
    __device__ __forceinline__ float at(int d) const {
        if constexpr (kDims == 0) {
            return row[d];
        } else {
            u32 v = 0;
#pragma unroll
            for (int i = 0; i < kDims; ++i) v |= __float_as_uint(p[i]) & (d == i ? ~0u : 0u);
            return __uint_as_float(v);
        }
    }
};

template <int kDims>
__device__ __forceinline__ float squared_distance(const Query<kDims>& q, const NodeRow<kDims>& node, int k) {
#pragma clang fp contract(off)
    float acc = 0.0f;  // 0 + t0*t0 is t0*t0 exactly
    if constexpr (kDims > 0) {
#pragma unroll
        for (int d = 0; d < kDims; ++d) {
            const float t = q.c[d] - node.p[d];
            acc = acc + t * t;
        }
    } else {
        for (int d = 0; d < k; ++d) {
            const float t = q.row[d] - node.row[d];
            acc = acc + t * t;
        }
    }
    return acc;
}

// The split offset q[split] - p[split] and (dist non-null) the squared
// distance, from the per-dimension differences computed once: the split
// one is picked by selects (the same subtraction, so the same value), which
// saves the masked picks of both coordinates. kDims == 0: read in place.
template <int kDims>
__device__ __forceinline__ float split_offset(const Query<kDims>& q, const NodeRow<kDims>& node, int split, int k,
                                              float* dist) {
#pragma clang fp contract(off)
    if constexpr (kDims > 0) {
        float t[kDims];
#pragma unroll
        for (int d = 0; d < kDims; ++d) t[d] = q.c[d] - node.p[d];
        float diff = t[0];
#pragma unroll
        for (int d = 1; d < kDims; ++d) diff = split == d ? t[d] : diff;
        if (dist) {
            float acc = 0.0f;  // as squared_distance: 0 + t0*t0 is t0*t0 exactly
#pragma unroll
            for (int d = 0; d < kDims; ++d) acc = acc + t[d] * t[d];
            *dist = acc;
        }
        return diff;
    } else {
        if (dist) *dist = squared_distance<kDims>(q, node, k);
        return q.at(split) - node.at(split);
    }
}

// The K best candidates as 64-bit keys (float bits of the squared distance,
// which order like the values for non-negative floats, then the index), in
// descending order: slot[0] is the K-th best. Slots K .. kK-1 hold 0, below
// every key, so they never move and the K best stay in slots 0 .. K-1.
template <int kK>
struct Best {
    u64 slot[kK];

    __device__ __forceinline__ void init(int K) {
#pragma unroll
        for (int i = 0; i < kK; ++i) slot[i] = i < K ? ~0ull : 0ull;
    }
    __device__ __forceinline__ u32 worst_bits() const { return (u32)(slot[0] >> 32); }
    // key < slot[0]: slot[0] leaves, the larger keys move up one, key enters
    __device__ __forceinline__ void insert(u64 key) {
        bool placed = false;
#pragma unroll
        for (int i = 0; i < kK - 1; ++i) {
            const u64 next = slot[i + 1];
            const bool up = !placed && next > key;
            slot[i] = up ? next : (placed ? slot[i] : key);
            placed = placed || !up;
        }
        if (!placed) slot[kK - 1] = key;
    }
};

// Writes query qi's result: its K keys ascending (slot K-1 first), or the
// hand-over mark.
template <int kK>
__device__ __forceinline__ void write_result(const KnnArgs& a, u64 qi, const Best<kK>& best, bool handed,
                                             u32 visits) {
    if (a.visits_out) a.visits_out[qi] = visits;
    int32_t* out_idx = a.idx_out + qi * (u64)a.K;
    if (handed) {
        const u32 b = best.worst_bits();
        out_idx[0] = b <= kInfBits ? kHandedOver - 1 - (int32_t)b : kHandedOver;
        return;
    }
    float* out_d2 = a.d2_out ? a.d2_out + qi * (u64)a.K : nullptr;
#pragma unroll
    for (int i = 0; i < kK; ++i) {
        if (i >= a.K) continue;
        const u64 key = best.slot[i];
        const int at = a.K - 1 - i;
        const bool empty = key == ~0ull;
        out_idx[at] = empty ? -1 : (int32_t)(u32)key;
        if (out_d2) out_d2[at] = empty ? __uint_as_float(0x7f800000u) : __uint_as_float((u32)(key >> 32));
    }
}

// First pass: one thread per query.
template <int kK, int kDims>
__global__ __launch_bounds__(kKnnBlock) void k_knn(KnnArgs a) {
    const u64 qi = (u64)blockIdx.x * kKnnBlock + threadIdx.x;
    if (qi >= (u64)a.q) return;
    Query<kDims> q;
    q.load(a.queries, qi, a.k);
    Best<kK> best;
    best.init(a.K);
    const u32 n = (u32)a.n;
    const int k = kDims > 0 ? kDims : a.k;
    u32 visits = 0;
    bool handed = false;
    if (n > 0) {
        // prev: the node the thread arrived from (~0 = from above the root)
        u32 curr = 0, prev = ~0u;
        int dim = 0;  // split dimension of curr's level
        // The split offsets (query - plane) of the nodes on the current path,
        // innermost first, for its deepest kPathRegs nodes: coming back up
        // to one of them needs no second load of its row.
        float path[kPathRegs];
        int held = 0;
        for (;;) {
            if (curr >= n) {  // a child that does not exist: back to its parent
                prev = curr;
                curr = (curr - 1) >> 1;
                dim = dim == 0 ? k - 1 : dim - 1;
                continue;
            }
            const u32 parent = curr == 0 ? ~0u : (curr - 1) >> 1;
            const u32 left = 2 * curr + 1;
            const int down = dim + 1 == k ? 0 : dim + 1;
            if (prev == parent) {
                // first visit: the node's point is a candidate; go to the
                // query's side first
                if (visits == a.budget) {
                    handed = true;
                    break;
                }
                ++visits;
                NodeRow<kDims> node;
                node.load(a.tree, curr, k);
                const int split = a.dims ? a.dims[curr] : dim;
                float dist;
                const float diff = split_offset<kDims>(q, node, split, k, &dist);
                const u32 bits = __float_as_uint(dist);
                if (bits <= best.worst_bits()) {
                    const u64 key = ((u64)bits << 32) | (u32)a.perm[curr];
                    if (key < best.slot[0]) best.insert(key);
                }
#pragma unroll
                for (int i = kPathRegs - 1; i > 0; --i) path[i] = path[i - 1];
                path[0] = diff;
                held = held < kPathRegs ? held + 1 : kPathRegs;
                prev = curr;
                curr = diff < 0.0f ? left : left + 1;
                dim = down;
                continue;
            }
            // back from a child: curr's offset, held or read again
            float diff;
            if (held > 0) {
                diff = path[0];
            } else {
                NodeRow<kDims> node;
                node.load(a.tree, curr, k);
                const int split = a.dims ? a.dims[curr] : dim;
                diff = split_offset<kDims>(q, node, split, k, nullptr);
                path[0] = diff;
                held = 1;
            }
            const u32 near = diff < 0.0f ? left : left + 1;
            const u32 far = diff < 0.0f ? left + 1 : left;
            if (prev == near && far < n && __float_as_uint(diff * diff) <= best.worst_bits()) {
                prev = curr;
                curr = far;
                dim = down;
                continue;
            }
            // leaving curr upwards
#pragma unroll
            for (int i = 0; i < kPathRegs - 1; ++i) path[i] = path[i + 1];
            --held;
            if (curr == 0) break;
            prev = curr;
            curr = parent;
            dim = dim == 0 ? k - 1 : dim - 1;
        }
    }
    write_result<kK>(a, qi, best, handed, visits);
}

__device__ __forceinline__ u32 wave_sum(u32 v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ int level_of32(u32 i) { return 31 - __clz(i + 1); }

__device__ __forceinline__ u64 read_lane64(u64 v, int lane) {
    const u32 lo = __builtin_amdgcn_readlane((u32)v, lane), hi = __builtin_amdgcn_readlane((u32)(v >> 32), lane);
    return ((u64)hi << 32) | lo;
}

// The K best keys of the wave's query so far, one per lane: lanes 0 .. K-1
// hold them in ascending order (~0 = empty), lanes K .. 63 are unused. Every
// lane's candidates go into the one list, so the pruning radius is the
// query's own K-th distance so far, or the cap if that is smaller: a key
// that K points the first pass examined are all at or below (so that the
// true K-th is too).
struct WaveBest {
    u64 key;   // this lane's slot
    u64 cap;   // a key known to be no better than the K-th (~0: none)
    u64 kth;   // min(slot K-1, cap), the same in every lane

    __device__ __forceinline__ void init(u64 bound) {
        key = ~0ull;
        cap = kth = bound;
    }
    __device__ __forceinline__ u32 worst_bits() const { return (u32)(kth >> 32); }
    // Inserts every lane's candidate c (~0: none), lowest lane first; each
    // one shifts the larger keys up one lane and drops slot K-1.
    __device__ __forceinline__ void insert_all(u64 c, int K) {
        const int lane = threadIdx.x & 63;
        u64 want = __ballot(c < kth);
        while (want) {
            const int src = __ffsll((long long)want) - 1;
            want &= want - 1;
            const u64 ck = read_lane64(c, src);
            if (ck >= kth) continue;  // (the K-th may have dropped below it meanwhile)
            const u32 pos = (u32)__popcll(__ballot(lane < K && key < ck));
            const u64 up = __shfl_up(key, 1, 64);
            key = (u32)lane < pos ? key : ((u32)lane == pos ? ck : up);
            const u64 last = read_lane64(key, K - 1);
            kth = last < cap ? last : cap;
        }
    }
};

// One lane's walk of a subtree by parent links (as in the first pass; it
// ends when it climbs back out of its root), advanced to its next candidate.
template <int kDims>
struct LaneWalk {
    u32 curr, prev, root;
    int dim;

    __device__ __forceinline__ void start(u32 c, int k) {
        root = c;
        curr = c;
        prev = c == 0 ? ~0u : (c - 1) >> 1;
        dim = level_of32(c) % k;
    }
    // Walks to the next node visited for the first time and sets *cand to its
    // key if its distance is within `worst` (else ~0); false when the walk
    // is over.
    __device__ __forceinline__ bool next(const KnnArgs& a, const Query<kDims>& q, u32 worst, int k, u64* cand) {
        const u32 n = (u32)a.n;
        for (;;) {
            if (curr >= n) {
                prev = curr;
                curr = (curr - 1) >> 1;
                dim = dim == 0 ? k - 1 : dim - 1;
                continue;
            }
            const u32 parent = curr == 0 ? ~0u : (curr - 1) >> 1;
            NodeRow<kDims> node;
            node.load(a.tree, curr, k);
            const int split = a.dims ? a.dims[curr] : dim;
            float dist;
            const float diff = split_offset<kDims>(q, node, split, k, &dist);
            const u32 left = 2 * curr + 1;
            const u32 near = diff < 0.0f ? left : left + 1;
            const u32 far = diff < 0.0f ? left + 1 : left;
            const int down = dim + 1 == k ? 0 : dim + 1;
            if (prev == parent) {
                const u32 bits = __float_as_uint(dist);
                *cand = bits <= worst ? ((u64)bits << 32) | (u32)a.perm[curr] : ~0ull;
                prev = curr;
                curr = near;
                dim = down;
                return true;
            }
            if (prev == near && far < n && __float_as_uint(diff * diff) <= worst) {
                prev = curr;
                curr = far;
                dim = down;
                continue;
            }
            if (curr == root) return false;
            prev = curr;
            curr = parent;
            dim = dim == 0 ? k - 1 : dim - 1;
        }
    }
};

// Second pass: every query the first pass handed over, searched by one
// 64-lane workgroup. Workgroup w owns queries [64w, 64w + 64). As in the
// first pass, a search goes down the near side of every plane first; here
// each lane follows one such path, one node a step, and leaves the far side
// of each plane it passes on a shared stack in LDS with a lower bound on its
// squared distance. A lane whose path ends takes the most recently left far
// side that is still within the (shared) K-th distance.
template <int kDims>
__global__ __launch_bounds__(64) void k_knn_wave(KnnArgs a) {
    __shared__ u64 stack[kWaveStack];  // (lower bound bits << 32) | node
    const int lane = threadIdx.x;
    const u64 base = (u64)blockIdx.x * 64;
    const u64 me = base + lane;
    const int32_t mark = me < (u64)a.q ? a.idx_out[me * (u64)a.K] : 0;
    const bool marked = mark <= kHandedOver;
    u64 todo = __ballot(marked);
    const u32 n = (u32)a.n;
    const int k = kDims > 0 ? kDims : a.k;
    constexpr u32 kNone = ~0u;
    while (todo) {
        const int owner = __ffsll((long long)todo) - 1;
        todo &= todo - 1;
        const u64 qi = base + owner;
        Query<kDims> q;
        q.load(a.queries, qi, a.k);
        // The first pass's K-th distance bounds the answer's: start from it.
        const int32_t owner_mark = __shfl(mark, owner, 64);
        WaveBest best;
        best.init(owner_mark == kHandedOver ? ~0ull : ((u64)(u32)(kHandedOver - 1 - owner_mark) << 32) | 0xffffffffu);
        u32 examined = 0, top = 0;
        // this lane's path: its next node and that node's bound
        u32 cur = lane == 0 && n > 0 ? 0u : kNone, cur_bound = 0;
        for (;;) {
            // lanes without a path take the most recent far sides
            const u64 idle = __ballot(cur == kNone);
            const u32 want = (u32)__popcll(idle);
            const u32 take = want < top ? want : top;
            if (take == 0 && want == 64) break;  // no path and no far side left
            if (cur == kNone) {
                const u32 r = (u32)__popcll(idle & ((1ull << lane) - 1));  // idle lanes below
                if (r < take) {
                    const u64 entry = stack[top - 1 - r];
                    cur = (u32)entry;
                    cur_bound = (u32)(entry >> 32);
                }
            }
            top -= take;
            __syncthreads();  // every pop read before pushes overwrite
            // one node of each path: a candidate, then the near side next
            u64 cand = ~0ull;
            float diff = 0.0f;
            bool live = cur != kNone && cur_bound <= best.worst_bits();
            if (live) {
                ++examined;
                NodeRow<kDims> row;
                row.load(a.tree, cur, k);
                const int dim = a.dims ? a.dims[cur] : level_of32(cur) % k;
                const u32 bits = __float_as_uint(squared_distance<kDims>(q, row, k));
                if (bits <= best.worst_bits()) cand = ((u64)bits << 32) | (u32)a.perm[cur];
                diff = q.at(dim) - row.at(dim);
            }
            best.insert_all(cand, a.K);
            const u32 worst = best.worst_bits();
            u64 push = 0;
            u32 npush = 0;
            if (live) {
                const u32 left = 2 * cur + 1;
                const u32 near = diff < 0.0f ? left : left + 1;
                const u32 far = diff < 0.0f ? left + 1 : left;
                const u32 db = __float_as_uint(diff * diff);
                const u32 far_bound = db > cur_bound ? db : cur_bound;
                if (far < n && far_bound <= worst) {
                    push = ((u64)far_bound << 32) | far;
                    npush = 1;
                }
                cur = near < n ? near : kNone;  // (its bound is cur_bound: checked next step)
            } else {
                cur = kNone;
            }
            // stack slots of the pushes: lanes in order
            const u64 pushers = __ballot(npush != 0);
            const u32 total = (u32)__popcll(pushers);
            if (top + total <= a.wave_stack) {
                if (npush) stack[top + (u32)__popcll(pushers & ((1ull << lane) - 1))] = push;
                top += total;
            } else {
                // No room: each such lane walks its far side itself, by
                // parent links, the wave inserting the candidates of every
                // step; its own path waits.
                LaneWalk<kDims> walk;
                bool walking = npush != 0;
                if (walking) walk.start((u32)push, k);
                while (__ballot(walking)) {
                    u64 c = ~0ull;
                    if (walking) {
                        if (walk.next(a, q, best.worst_bits(), k, &c)) ++examined;
                        else walking = false;
                    }
                    best.insert_all(c, a.K);
                }
            }
            __syncthreads();
        }
        // the list is in lane order: lane i holds the (i+1)-th neighbour
        if (lane < a.K) {
            const bool empty = best.key == ~0ull;
            a.idx_out[qi * (u64)a.K + lane] = empty ? -1 : (int32_t)(u32)best.key;
            if (a.d2_out)
                a.d2_out[qi * (u64)a.K + lane] = empty ? __uint_as_float(0x7f800000u)
                                                       : __uint_as_float((u32)(best.key >> 32));
        }
        const u32 all = wave_sum(examined);
        if (lane == 0 && a.visits_out) a.visits_out[qi] += all;
        __syncthreads();
    }
}

template <int kK>
void launch_knn(const KnnArgs& a, hipStream_t stream) {
    const unsigned grid = (unsigned)((a.q + kKnnBlock - 1) / kKnnBlock);
    const unsigned waves = (unsigned)((a.q + 63) / 64);
    switch (a.k) {
        case 2:
            k_knn<kK, 2><<<grid, kKnnBlock, 0, stream>>>(a);
            k_knn_wave<2><<<waves, 64, 0, stream>>>(a);
            break;
        case 3:
            k_knn<kK, 3><<<grid, kKnnBlock, 0, stream>>>(a);
            k_knn_wave<3><<<waves, 64, 0, stream>>>(a);
            break;
        case 4:
            k_knn<kK, 4><<<grid, kKnnBlock, 0, stream>>>(a);
            k_knn_wave<4><<<waves, 64, 0, stream>>>(a);
            break;
        default:
            k_knn<kK, 0><<<grid, kKnnBlock, 0, stream>>>(a);
            k_knn_wave<0><<<waves, 64, 0, stream>>>(a);
            break;
    }
}

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
    if (!a || !b || an == 0 || bn == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + bn && y < x + an;
}

kdt_status knn_impl(const float* tree, const int32_t* perm, const int32_t* dims, int64_t N, int32_t k,
                    const float* queries, int64_t Q, int32_t K, int32_t* idx_out, float* d2_out,
                    uint32_t* visits_out, uint32_t budget, uint32_t wave_stack, hipStream_t stream) {
    if (N < 0 || N > INT32_MAX || k < 1 || k > 65535 || Q < 0 || Q > INT32_MAX || K < 1 ||
        K > kKnnMaxK || wave_stack < 1 || wave_stack > (uint32_t)kWaveStack)
        return KDT_ERR_INVALID_ARG;
    if (Q == 0) return KDT_OK;
    if (!queries || !idx_out || (N > 0 && (!tree || !perm))) return KDT_ERR_INVALID_ARG;
    const size_t tree_b = (size_t)N * k * sizeof(float), perm_b = (size_t)N * sizeof(int32_t);
    const size_t q_b = (size_t)Q * k * sizeof(float), out_b = (size_t)Q * K * sizeof(int32_t);
    const void* ins[4] = {tree, perm, queries, dims};
    const size_t in_b[4] = {tree_b, perm_b, q_b, dims ? perm_b : 0};
    for (int i = 0; i < 4; ++i)
        if (overlap(idx_out, out_b, ins[i], in_b[i]) || overlap(d2_out, out_b, ins[i], in_b[i]))
            return KDT_ERR_INVALID_ARG;
    const size_t v_b = (size_t)Q * sizeof(uint32_t);
    for (int i = 0; i < 4; ++i)
        if (overlap(visits_out, v_b, ins[i], in_b[i])) return KDT_ERR_INVALID_ARG;
    if (overlap(idx_out, out_b, d2_out, out_b) || overlap(visits_out, v_b, idx_out, out_b) ||
        overlap(visits_out, v_b, d2_out, out_b))
        return KDT_ERR_INVALID_ARG;
    KnnArgs a{tree, perm, dims, N, k, queries, Q, K, idx_out, d2_out, visits_out, budget, wave_stack};
    if (K <= 1) launch_knn<1>(a, stream);
    else if (K <= 2) launch_knn<2>(a, stream);
    else if (K <= 4) launch_knn<4>(a, stream);
    else if (K <= 8) launch_knn<8>(a, stream);
    else if (K <= 16) launch_knn<16>(a, stream);
    else launch_knn<32>(a, stream);
    return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
}

}  // namespace

extern "C" kdt_status kdt_knn(const float* tree, const int32_t* perm, const int32_t* dims, int64_t N,
                              int32_t k, const float* queries, int64_t Q, int32_t K, int32_t* idx_out,
                              float* d2_out, uint32_t* visits_out, hipStream_t stream) {
    return knn_impl(tree, perm, dims, N, k, queries, Q, K, idx_out, d2_out, visits_out,
                    default_budget(K), kWaveStack, stream);
}

extern "C" kdt_status kdt_knn_budget(const float* tree, const int32_t* perm, const int32_t* dims,
                                     int64_t N, int32_t k, const float* queries, int64_t Q, int32_t K,
                                     int32_t* idx_out, float* d2_out, uint32_t* visits_out,
                                     uint32_t budget, hipStream_t stream) {
    return knn_impl(tree, perm, dims, N, k, queries, Q, K, idx_out, d2_out, visits_out, budget, kWaveStack,
                    stream);
}

extern "C" kdt_status kdt_knn_debug(const float* tree, const int32_t* perm, const int32_t* dims,
                                    int64_t N, int32_t k, const float* queries, int64_t Q, int32_t K,
                                    int32_t* idx_out, float* d2_out, uint32_t* visits_out,
                                    uint32_t budget, uint32_t wave_stack, hipStream_t stream) {
    return knn_impl(tree, perm, dims, N, k, queries, Q, K, idx_out, d2_out, visits_out,
                    budget == 0xffffffffu ? default_budget(K) : budget, wave_stack, stream);
}
