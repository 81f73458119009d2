// Left-balanced k-d tree build for MI355X (gfx950): the tag-based
// "trickle-down" construction of I. Wald, "GPU-friendly, Parallel, and
// (Almost-)In-Place Construction of Left-Balanced k-d Trees" (arXiv
// 2211.00120), cited as [W] with the paragraph that states each fact.
//
// Round l of [W] sorts every point by (tag, coordinate l mod k, original
// index) and refines every tag from its sorted position. Here that sort is a
// stable LSD radix sort from index order with 8-bit digits. Its first
// passes, over the coordinate's bytes, do not depend on the tags: they always
// produce the points ordered by (coordinate d, index), whatever the round.
// That order is computed once per split dimension ("presort") and every
// round then runs only its tag-digit passes over it; the last tag pass
// updates the tags in place from the sorted positions.
//
// Pipeline per build (all on the caller's stream, nothing allocated):
//   k_init       AoS points -> one column per split dimension.
//   4 passes     per dimension: stable sort of (key(x_d), index) -> order_d
//                (the points by coordinate d, then index); the last pass
//                also writes the inverse, rank_d[order_d[r]] = r. Dimensions
//                d >= 1 carry rank_(d+1) as a second payload, which lands as
//                next_d.
//   k_cross      next_0[r] = position in order_1 of the r-th point of
//                order_0 (all writes; no random reads).
//   k_round0     round 0 (all tags 0): tags straight from order_0.
//   per round l = 1 .. l0-1, d = l mod k:
//     1-2 passes stable sort by tag of the records (tag, next_d) kept in
//                order_d order; the last one computes each point's new tag
//                and writes it where round l+1 reads it (tags are kept in
//                the order of the dimension that reads them), or, in round
//                l0-1, writes the sorted point indices for the next stage.
//   k_place_top  nodes above level l0.
//   k_subtree    one workgroup per level-l0 subtree (<= 4096 points) runs
//                that subtree's remaining rounds in LDS and writes its
//                level-order output.
//
// A radix pass is reduce-then-scan: digit counts of each tile (LDS
// atomics), a scan of the per-chunk counts per digit that also yields the
// digit totals, and a scatter that ranks each tile (wave64 ballots, stable
// multi-split), places it from those counts and stages it in LDS so that the
// global writes of one digit are contiguous. No workgroup ever waits on
// another.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kdt.h"

namespace {

typedef uint8_t u8;
typedef uint32_t u32;
typedef uint64_t u64;
typedef int64_t i64;

constexpr int kRadixBits = 8;
constexpr int kRadix = 1 << kRadixBits;
constexpr int kBlock = 256;                // threads per workgroup
constexpr int kWaves = kBlock / 64;        // wave64
constexpr int kItems = 16;                 // records per thread in a radix tile
constexpr int kTile = kBlock * kItems;     // records per radix tile
constexpr int kKeyBytes = 4;               // order-preserving coordinate key
constexpr int kChunkTiles = 4;             // tiles per digit-count chunk
static_assert(kBlock == kRadix, "the tile kernels map one thread to one digit");
static_assert(kBlock * kChunkTiles <= 1024, "one workgroup counts a whole chunk");

// ------------------------------------------------------------ tree geometry
// Level-order complete tree with N nodes ([W], indexing paragraph):
// level(i) = floor(log2(i+1)), numLevels(N) = level(N-1)+1, F(l) = 2^l - 1.

struct Geometry {
    i64 n;      // nodes (= points)
    int levels; // L = numLevels(N)
    i64 last;   // nodes on the last level: N - F(L-1)
};

__host__ __device__ inline int level_of(u64 i) { return 63 - __builtin_clzll(i + 1); }
__host__ __device__ inline u64 full_nodes(int l) { return (1ull << l) - 1; }

__host__ __device__ inline Geometry make_geometry(i64 n) {
    Geometry g;
    g.n = n;
    g.levels = level_of((u64)(n - 1)) + 1;
    g.last = n - (i64)full_nodes(g.levels - 1);
    return g;
}

// Size of the subtree rooted at s ([W], sb/ss paragraph; the closed form is
// not in the extracted text and is derived here): the dd = L-1-level(s)
// levels below s's own are full (2^dd - 1 nodes), and of the 2^dd
// last-level slots under s, which start at id (s+1)*2^dd - 1, only those
// below N exist.
__host__ __device__ inline u64 subtree_size(const Geometry& g, u64 s) {
    if (s >= (u64)g.n) return 0;
    int dd = g.levels - 1 - level_of(s);
    u64 span = 1ull << dd;
    i64 first_last = (i64)((s + 1) << dd) - 1;
    i64 extra = g.n - first_last;
    if (extra < 0) extra = 0;
    if (extra > (i64)span) extra = (i64)span;
    return (span - 1) + (u64)extra;
}

// First sorted position of subtree s (on level l) in the round that fixes
// level l ([W], sb/ss paragraph; derived): the F(l) nodes above level l are
// already fixed and sort first in tag order, then the j = s - F(l) subtrees
// left of s on level l, each with 2^dd - 1 full-level nodes, plus the
// last-level nodes under them, min(M, j * 2^dd).
__host__ __device__ inline u64 segment_begin(const Geometry& g, u64 s, int l) {
    u64 j = s - full_nodes(l);
    int dd = g.levels - 1 - l;
    u64 under = j << dd;
    if (under > (u64)g.last) under = (u64)g.last;
    return full_nodes(l) + j * ((1ull << dd) - 1) + under;
}

// Order-preserving map of float bits to unsigned: IEEE order with -0 == +0.
// Pure bit tests, so denormals are never flushed.
__device__ inline u32 float_key(u32 b) {
    if ((b & 0x7fffffffu) == 0) return 0x80000000u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ------------------------------------------------------------- block scans

__device__ inline u32 wave_inclusive_scan(u32 v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        u32 t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Exclusive scan of one value per thread across the workgroup.
__device__ inline u32 block_exclusive_scan(u32 v, u32* s_wave) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    u32 inc = wave_inclusive_scan(v);
    if (lane == 63) s_wave[w] = inc;
    __syncthreads();
    u32 off = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i)
        if (i < w) off += s_wave[i];
    __syncthreads();
    return off + inc - v;
}

__device__ inline u64 wave_inclusive_scan64(u64 v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        u64 t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Exclusive scan of one 64-bit value per thread across the workgroup (used
// for two 32-bit scans at once whose sums cannot carry out of 32 bits).
__device__ inline u64 block_exclusive_scan64(u64 v, u64* s_wave) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    u64 inc = wave_inclusive_scan64(v);
    if (lane == 63) s_wave[w] = inc;
    __syncthreads();
    u64 off = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i)
        if (i < w) off += s_wave[i];
    __syncthreads();
    return off + inc - v;
}

// Radix passes over the tag in round l >= 1: only the 2^l live tags
// F(l) .. F(l+1)-1 are sorted, by their offset from F(l) (l bits).
__host__ __device__ inline int tag_passes(int l) { return (l + kRadixBits - 1) / kRadixBits; }

// ------------------------------------------------------ global-phase kernels

// Column copy of the split dimensions.
__global__ __launch_bounds__(kBlock) void k_init(const float* __restrict__ pts, i64 n, int k,
                                                 int kcols, float* __restrict__ cols) {
    const i64 stride = (i64)gridDim.x * kBlock;
    for (i64 e = (i64)blockIdx.x * kBlock + threadIdx.x; e < n; e += stride) {
        const float* row = pts + e * k;
        for (int d = 0; d < kcols; ++d) cols[(i64)d * n + e] = row[d];
    }
}

// next[rank_d[i]] = rank_e[i]: for the r-th point of order_d, its position
// in order_e. Reads both ranks in index order, writes scattered.
__global__ __launch_bounds__(kBlock) void k_cross(const u32* __restrict__ rank_d,
                                                  const u32* __restrict__ rank_e, i64 n,
                                                  u32* __restrict__ next) {
    const i64 stride = (i64)gridDim.x * kBlock;
    for (i64 i = (i64)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        const u32 r = rank_d[i];
        if (r < (u64)n) next[r] = rank_e[i];
    }
}

// Round 0: every tag is 0, so the sorted order is order_0 itself and the
// pivot sits at position |S(1)|. Writes each point's new tag at its
// position in the order round 1 reads.
__global__ __launch_bounds__(kBlock) void k_round0(const u32* __restrict__ next, Geometry geo,
                                                   u32* __restrict__ tag_next) {
    const u64 pivot = subtree_size(geo, 1);
    const i64 stride = (i64)gridDim.x * kBlock;
    for (i64 r = (i64)blockIdx.x * kBlock + threadIdx.x; r < geo.n; r += stride) {
        const u32 q = next[r];
        if (q < (u64)geo.n) tag_next[q] = (u64)r < pivot ? 1u : ((u64)r > pivot ? 2u : 0u);
    }
}

// Tags after some rounds, back in original index order (diagnostics only).
__global__ __launch_bounds__(kBlock) void k_unpermute(const u32* __restrict__ tagq,
                                                      const u32* __restrict__ order, i64 n,
                                                      u32* __restrict__ out) {
    const i64 stride = (i64)gridDim.x * kBlock;
    for (i64 r = (i64)blockIdx.x * kBlock + threadIdx.x; r < n; r += stride) {
        const u32 i = order[r];
        if (i < (u64)n) out[i] = tagq ? tagq[r] : 0u;
    }
}

enum Src { kSrcColumn = 0, kSrcArrays = 1 };
enum Sink { kSinkArrays = 0, kSinkVals = 1, kSinkTags = 2 };

// One stable radix pass over n (key, val) records is three launches
// (reduce-then-scan; no workgroup ever waits on another):
//   k_tile_count  digit counts of every tile of kTile records,
//   k_tile_scan   per digit, exclusive scan over the tiles plus the digit's
//                 first slot -> the first global slot of (tile, digit),
//   k_tile_scatter rank each tile again and move its records there.
struct PassArgs {
    i64 n;                     // records of this pass
    i64 n_all;                 // points (bound of tag_out and fixed_*)
    int shift;                 // digit = ((key - key_base) >> shift) & 255
    u32 key_base;              // records with key < key_base are fixed: they
                               //   are not sorted and go to a fixed_* array
    const float* col;          // kSrcColumn: key = key(col[i]), val = i
    const u32* keys_in;        // kSrcArrays
    const u32* vals_in;        // kSrcArrays
    u32* keys_out;             // kSinkArrays
    u32* vals_out;             // kSinkArrays, kSinkVals
    u32* tag_out;              // kSinkTags: tag_out[val] = the record's new tag
    u32* rank_out;             // kSinkVals, optional: rank_out[val] = val's slot
    const u32* extra_in;       // optional second payload (nullptr: none); with
    u32* extra_out;            //   kSrcColumn it is indexed by point index
    u32* digit_totals;         // 256 counts of this pass's digit over all records
    u32* tile_counts;          // tiles x 256: digit counts of each tile
    u32* chunk_slots;          // chunks x 256: digit counts of each chunk of
                               //   kChunkTiles tiles, then the counts of the
                               //   digit in the chunks before it
    u32* fixed_tags;           // fixed record: fixed_tags[val] = key (its tag)
    u32* fixed_vals;           // fixed record: fixed_vals[key] = val (node key
                               //   sits at sorted position key)
    Geometry geo;              // kSinkTags
    int round;                 // kSinkTags
};

// Records of item j of this thread: wave w owns kItems rows of 64
// consecutive records of the tile.
template <int kSrc>
__device__ inline void load_tile(const PassArgs& a, i64 wbase, u32 (&key)[kItems],
                                 u32 (&val)[kItems]) {
    // (the optional second payload is loaded by the scatter kernel itself)
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const i64 e = wbase + (i64)j * 64;
        key[j] = 0;
        val[j] = 0;
        if (e < a.n) {
            if (kSrc == kSrcColumn) {
                key[j] = float_key(__float_as_uint(a.col[e]));
                val[j] = (u32)e;
            } else {
                key[j] = a.keys_in[e];
                val[j] = a.vals_in[e];
            }
        }
    }
}

// Rank inside the wave: lanes holding the same digit are found with eight
// ballots (a lane's peers are the lanes that never disagree with it on a
// bit: the OR over bits of vote ^ own-bit-mask, inverted); the lowest such
// lane bumps the wave's counter for the digit. rank[j] = records of the
// same digit earlier in the wave's rows. Records past the end, and with
// kTags those whose key (an offset from F(l)) wrapped below zero (fixed
// points), are not ranked.
template <bool kTags>
__device__ inline void wave_rank(const u32 (&key)[kItems], i64 wbase, i64 n, int shift,
                                 u32* count, u32 (&rank)[kItems]) {
    const int lane = threadIdx.x & 63;
    for (int i = lane; i < kRadix; i += 64) count[i] = 0;
    const u64 below = (1ull << lane) - 1;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const bool valid = (wbase + (i64)j * 64) < n && (!kTags || (int)key[j] >= 0);
        const u32 d = (key[j] >> shift) & (kRadix - 1);
        u32 miss_lo = 0, miss_hi = 0;
#pragma unroll
        for (int b = 0; b < kRadixBits; ++b) {
            const u64 vote = __ballot((d >> b) & 1);
            const u32 m = (u32)((int)(d << (31 - b)) >> 31);  // all ones where the bit is set
            miss_lo |= (u32)vote ^ m;
            miss_hi |= (u32)(vote >> 32) ^ m;
        }
        const u64 peers = __ballot(valid) & ~(((u64)miss_hi << 32) | miss_lo);
        const u32 before = __popcll(peers & below);
        u32 seen = 0;
        if (valid) seen = count[d];
        rank[j] = seen + before;
        if (valid && before == 0) count[d] = seen + (u32)__popcll(peers);
    }
}

// Keys of item j of this thread (the same record layout as load_tile).
template <int kSrc>
__device__ inline void load_keys(const PassArgs& a, i64 wbase, u32 (&key)[kItems]) {
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const i64 e = wbase + (i64)j * 64;
        key[j] = 0;
        if (e < a.n)
            key[j] = kSrc == kSrcColumn ? float_key(__float_as_uint(a.col[e])) : a.keys_in[e];
    }
}

// Digit counts of kChunkTiles consecutive tiles: one row per tile and the
// chunk's total (fixed records are not counted). Each group of kBlock threads counts one tile (the same
// record layout as the scatter's tiles), all tiles of the chunk at once.
// Counting needs no ranks, only LDS atomics; each thread merges runs of
// equal digits among its own records first, which keeps the skewed high
// bytes of clustered keys from piling onto one counter.
constexpr int kCountBlock = kBlock * kChunkTiles;
template <int kSrc>
__global__ __launch_bounds__(kCountBlock) void k_tile_count(PassArgs a) {
    __shared__ u32 hist[kCountBlock / 64][kRadix];
    __shared__ u32 rows[kChunkTiles][kRadix];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int g = tid / kBlock;  // tile of the chunk this thread counts
    const int gw = w % kWaves;   // wave within that tile
    const i64 t = (i64)blockIdx.x * kChunkTiles + g;
    const i64 wbase = t * kTile + (i64)gw * (64 * kItems) + lane;
    u32 key[kItems];
    load_keys<kSrc>(a, wbase, key);
    for (int i = lane; i < kRadix; i += 64) hist[w][i] = 0;  // this wave's own row
    u32 last = 0, run = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        if (wbase + (i64)j * 64 >= a.n) break;
        if (key[j] < a.key_base) continue;  // fixed: not sorted
        const u32 d = ((key[j] - a.key_base) >> a.shift) & (kRadix - 1);
        if (run && d != last) {
            atomicAdd(&hist[w][last], run);
            run = 0;
        }
        last = d;
        ++run;
    }
    if (run) atomicAdd(&hist[w][last], run);
    __syncthreads();
    const int d = tid % kRadix;
    u32 total = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) total += hist[g * kWaves + v][d];
    const i64 tiles = (a.n + kTile - 1) / kTile;
    if (t < tiles) a.tile_counts[(u64)t * kRadix + d] = total;
    rows[g][d] = total;
    __syncthreads();
    if (tid < kRadix) {
        u32 sum = 0;
#pragma unroll
        for (int c = 0; c < kChunkTiles; ++c) sum += rows[c][tid];
        a.chunk_slots[(u64)blockIdx.x * kRadix + tid] = sum;
    }
}

// One workgroup per digit d: slots[c][d] = counts of d in the chunks before
// c; totals[d] = all counts of d. Each thread scans a contiguous run of up
// to kScanRun chunks held in registers (one batch of loads); longer inputs
// loop over runs.
constexpr int kScanRun = 16;
__global__ __launch_bounds__(kBlock) void k_tile_scan(u32* __restrict__ slots, i64 chunks,
                                                      u32* __restrict__ totals) {
    __shared__ u32 s_wave[kWaves];
    __shared__ u32 s_carry;
    const int tid = threadIdx.x, d = blockIdx.x;
    if (tid == kBlock - 1) s_carry = 0;
    for (i64 t0 = 0; t0 < chunks; t0 += (i64)kBlock * kScanRun) {
        const i64 mine = t0 + (i64)tid * kScanRun;
        u32 v[kScanRun], sum = 0;
#pragma unroll
        for (int i = 0; i < kScanRun; ++i) {
            v[i] = mine + i < chunks ? slots[(u64)(mine + i) * kRadix + d] : 0u;
            sum += v[i];
        }
        __syncthreads();  // s_carry written
        const u32 carry = s_carry;
        u32 off = block_exclusive_scan(sum, s_wave) + carry;
        if (tid == kBlock - 1) s_carry = off + sum;
#pragma unroll
        for (int i = 0; i < kScanRun; ++i) {
            if (mine + i < chunks) slots[(u64)(mine + i) * kRadix + d] = off;
            off += v[i];
        }
    }
    __syncthreads();
    if (tid == 0) totals[d] = s_carry;
}

// kTags: a tag pass, whose records below key_base are fixed (not sorted).
template <int kSrc, int kSink, bool kExtra, bool kTags>
__global__ __launch_bounds__(kBlock) void k_tile_scatter(PassArgs a) {
    __shared__ union {
        u32 count[kWaves][kRadix];  // ranking: per-wave digit counts, then prefixes
        u32 keys[kTile];            // staging of the sorted tile
        u32 vals[kTile];
        u64 pairs[kExtra && kSink == kSinkVals ? kTile : 1];  // value + second payload
    } sm;
    __shared__ u8 s_digit[kTile];
    __shared__ u32 s_local[kRadix];  // first tile-local slot of each digit
    __shared__ u32 s_base[kRadix];   // global slot of tile-local slot 0 of each digit
    __shared__ u64 s_wave[kWaves];
    __shared__ u32 s_live;           // records of the tile that are sorted

    const int tid = threadIdx.x, w = tid >> 6;
    const i64 base = (i64)blockIdx.x * kTile;
    const i64 wbase = base + (i64)w * (64 * kItems) + (tid & 63);
    u32 key[kItems], val[kItems], rank[kItems], extra[kItems];
    load_tile<kSrc>(a, wbase, key, val);
    // First global slot of digit tid in this tile: where the digit starts in
    // the output, plus its counts in earlier chunks and in the chunk's
    // earlier tiles.
    const u32 digit_total = a.digit_totals[tid];
    const i64 chunk = blockIdx.x / kChunkTiles;
    u32 global_start = a.chunk_slots[(u64)chunk * kRadix + tid];
#pragma unroll
    for (int c = 0; c < kChunkTiles - 1; ++c) {
        const i64 t = chunk * kChunkTiles + c;
        if (t < (i64)blockIdx.x) global_start += a.tile_counts[(u64)t * kRadix + tid];
    }
    if (kExtra) {
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const i64 e = wbase + (i64)j * 64;
            extra[j] = e < a.n ? a.extra_in[e] : 0u;
        }
    }
    // Tag passes work on the offset of the tag from F(l): live tags map to
    // 0 .. 2^l - 1 and fixed ones wrap to values >= 2^31.
    const u32 kbase = kTags ? a.key_base : 0u;
    if (kTags) {
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            key[j] -= kbase;
            if ((wbase + (i64)j * 64) >= a.n || (int)key[j] >= 0) continue;
            // A fixed record goes straight to its final place: its tag for
            // the next round, or its node's slot of the sorted order.
            const u32 s = key[j] + kbase;  // the fixed node's id
            if (a.fixed_tags) {
                if (val[j] < (u64)a.n_all) a.fixed_tags[val[j]] = s;
            } else if (a.fixed_vals) {
                if (s < (u64)a.n_all) a.fixed_vals[s] = val[j];
            }
        }
    }
    wave_rank<kTags>(key, wbase, a.n, a.shift, sm.count[w], rank);
    __syncthreads();

    // Thread tid owns digit tid: per-wave prefixes and the tile total.
    u32 agg = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        const u32 c = sm.count[v][tid];
        sm.count[v][tid] = agg;
        agg += c;
    }
    // Both exclusive scans at once: digit totals (high word) and the tile's
    // digit counts (low word, at most kTile in all).
    const u64 starts = block_exclusive_scan64(((u64)digit_total << 32) | agg, s_wave);
    const u32 local_start = (u32)starts;
    global_start += (u32)(starts >> 32);
    s_local[tid] = local_start;
    s_base[tid] = global_start - local_start;  // modular; base + slot < n
    if (tid == kBlock - 1) s_live = local_start + agg;

    // (recomputed where needed rather than held in registers)
    auto live = [&](int j) { return (wbase + (i64)j * 64) < a.n && (!kTags || (int)key[j] >= 0); };
    auto digit = [&](int j) { return (key[j] >> a.shift) & (kRadix - 1); };
#pragma unroll
    for (int j = 0; j < kItems; ++j)
        if (live(j)) rank[j] += sm.count[w][digit(j)];
    __syncthreads();  // s_local written

    if (kSink == kSinkTags) {
        // Tag update ([W], tag and sort-order paragraphs): a point of subtree
        // s (s on level l, so s >= F(l)) at sorted position p moves to the
        // left child if p is before the pivot, to the right child if after,
        // and stays as node s if it is the pivot; pivot = start of s's
        // segment + size of the left subtree. Tags < F(l) are final (carried
        // over above). Those F(l) fixed points sort first, one per node id,
        // so the live ones, ranked here, start at position F(l).
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            if (!live(j)) continue;  // fixed ones are written already
            const u64 s = (u32)(key[j] + kbase);
            const u32 d = digit(j);
            const u64 p = (u64)kbase + (u32)(s_base[d] + s_local[d] + rank[j]);
            const u64 pivot = segment_begin(a.geo, s, a.round) + subtree_size(a.geo, 2 * s + 1);
            const u64 t = p < pivot ? 2 * s + 1 : (p > pivot ? 2 * s + 2 : s);
            if (val[j] < (u64)a.n_all) a.tag_out[val[j]] = (u32)t;
        }
        return;
    }

    const int valid_here = (int)s_live;
    // rank[j] becomes the record's slot in the tile's sorted order.
#pragma unroll
    for (int j = 0; j < kItems; ++j)
        if (live(j)) rank[j] += s_local[digit(j)];
    if (kSink == kSinkArrays) {
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            if (!live(j)) continue;
            sm.keys[rank[j]] = key[j] + kbase;
            s_digit[rank[j]] = (u8)digit(j);
        }
        __syncthreads();
        for (int i = tid; i < valid_here; i += kBlock) {
            const u32 dst = s_base[s_digit[i]] + (u32)i;
            if (dst < (u64)a.n) a.keys_out[dst] = sm.keys[i];
        }
        __syncthreads();
    }
    // Values; the optional second payload shares the value's 64-bit slot
    // when they are the only outputs, else it gets a staging round of its own.
    constexpr bool kPairs = kExtra && kSink == kSinkVals;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        if (!live(j)) continue;
        if (kPairs) sm.pairs[rank[j]] = ((u64)extra[j] << 32) | val[j];
        else sm.vals[rank[j]] = val[j];
        if (kSink == kSinkVals) s_digit[rank[j]] = (u8)digit(j);
    }
    __syncthreads();
    for (int i = tid; i < valid_here; i += kBlock) {
        const u32 dst = s_base[s_digit[i]] + (u32)i;
        if (dst >= (u64)a.n) continue;
        u32 v;
        if (kPairs) {
            const u64 pv = sm.pairs[i];
            v = (u32)pv;
            a.extra_out[dst] = (u32)(pv >> 32);
        } else {
            v = sm.vals[i];
        }
        a.vals_out[dst] = v;
        // The inverse permutation, written where the records are placed.
        if (kSink == kSinkVals && a.rank_out && v < (u64)a.n_all) a.rank_out[v] = dst;
    }
    if (kExtra && !kPairs) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            if (!live(j)) continue;
            sm.vals[rank[j]] = extra[j];
        }
        __syncthreads();
        for (int i = tid; i < valid_here; i += kBlock) {
            const u32 dst = s_base[s_digit[i]] + (u32)i;
            if (dst < (u64)a.n) a.extra_out[dst] = sm.vals[i];
        }
    }
}

// --------------------------------------------- subtrees finished in LDS
// Once every subtree on some level l0 holds at most kLocalMax points, the
// remaining rounds of each subtree only ever compare points of that subtree:
// a point's sorted position inside its segment, and therefore its next tag,
// depends on its own segment alone. One workgroup then runs those rounds for
// one subtree -- the same sort by (tag, coordinate, index) and the same tag
// update, with subtree-local tags and positions -- entirely in LDS, and
// writes the subtree's level-order output. The subtree rooted at global node
// c is itself the complete left-balanced tree of |S(c)| nodes (its share of
// the last level is a left-aligned run), so its local geometry is
// make_geometry(|S(c)|) and local node j on local level t is global node
// (c+1)*2^t - 1 + (j - F(t)).

constexpr int kLocalBlock = 512;                      // threads per subtree workgroup
constexpr int kLocalWaves = kLocalBlock / 64;
constexpr int kLocalItems = 8;                        // records per thread
constexpr int kLocalMax = kLocalBlock * kLocalItems;  // points per subtree
constexpr int kCachedDims = 3;                        // sorted orders kept in LDS
constexpr int kRowRegs = 4;                           // row loads batched up to this k
constexpr int kRowBatch = 4;                          // items whose rows load together
static_assert(kLocalBlock >= kRadix, "one thread per digit");

struct LocalShared {
    u32 exch[kLocalMax];                  // record exchange of the radix passes
    uint16_t count[kLocalWaves][kRadix];  // per-wave digit counters, then prefixes
    u32 start[kRadix];                    // first slot of each digit
    u32 wave[kLocalWaves];
    u64 reduce[2][kLocalWaves];           // AND / OR of the keys, per wave
    uint16_t tag[kLocalMax];              // local tag of each point (by index rank)
    uint16_t order[kCachedDims][kLocalMax];  // points sorted by (coordinate, index)
};

// The tag rounds keep per-wave segment counters in the exchange buffer: at
// local level t there are 2^t segments, t <= 11 for kLocalMax points, and
// 8-bit counters for 2048 segments must fit.
static_assert(kLocalWaves * (kLocalMax / 2) <= sizeof(LocalShared::exch), "round counters");

// Slot of item j of this thread: each wave owns kLocalItems rows of 64.
__device__ inline int local_slot(int j) {
    return (threadIdx.x >> 6) * (64 * kLocalItems) + j * 64 + (threadIdx.x & 63);
}

__device__ inline u32 local_exclusive_scan(u32 v, u32* s_wave) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    u32 inc = wave_inclusive_scan(v);
    if (lane == 63) s_wave[w] = inc;
    __syncthreads();
    u32 off = 0;
#pragma unroll
    for (int i = 0; i < kLocalWaves; ++i)
        if (i < w) off += s_wave[i];
    __syncthreads();
    return off + inc - v;
}

// Mask of key bits on which the records (all of the workgroup's valid
// ones) disagree; a radix pass over a byte outside it would not move
// anything and is skipped.
__device__ u64 local_varying_bits(const u64 (&rec)[kLocalItems], u32 nc, LocalShared& sh) {
    u64 all_and = ~0ull, all_or = 0;
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j)
        if ((u32)local_slot(j) < nc) {
            all_and &= rec[j];
            all_or |= rec[j];
        }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        all_and &= __shfl_xor(all_and, o, 64);
        all_or |= __shfl_xor(all_or, o, 64);
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sh.reduce[0][w] = all_and;
        sh.reduce[1][w] = all_or;
    }
    __syncthreads();
    u64 a = ~0ull, b = 0;
#pragma unroll
    for (int v = 0; v < kLocalWaves; ++v) {
        a &= sh.reduce[0][v];
        b |= sh.reduce[1][v];
    }
    __syncthreads();
    return a ^ b;
}

// One stable pass over all kLocalMax records of the workgroup by the 8-bit
// digit at `shift`. Unused slots hold all-ones records: they sit at the end
// and keep digit 255, so they stay behind every real record.
__device__ void local_pass(u64 (&rec)[kLocalItems], int shift, LocalShared& sh) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = lane; i < kRadix; i += 64) sh.count[w][i] = 0;
    const u64 below = (1ull << lane) - 1;
    // Rank inside the wave: lanes holding the same digit are found with eight
    // ballots; the lowest such lane bumps the wave's counter for the digit.
    u32 rank[kLocalItems];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 d = (u32)(rec[j] >> shift) & (kRadix - 1);
        u32 miss_lo = 0, miss_hi = 0;
#pragma unroll
        for (int b = 0; b < kRadixBits; ++b) {
            const u64 vote = __ballot((d >> b) & 1);
            const u32 m = (u32)((int)(d << (31 - b)) >> 31);  // all ones where the bit is set
            miss_lo |= (u32)vote ^ m;
            miss_hi |= (u32)(vote >> 32) ^ m;
        }
        const u64 peers = ~(((u64)miss_hi << 32) | miss_lo);
        const u32 before = __popcll(peers & below);
        const u32 seen = sh.count[w][d];
        rank[j] = seen + before;
        if (before == 0) sh.count[w][d] = seen + (u32)__popcll(peers);
    }
    __syncthreads();
    u32 agg = 0;
    if (tid < kRadix) {
#pragma unroll
        for (int v = 0; v < kLocalWaves; ++v) {
            const u32 c = sh.count[v][tid];
            sh.count[v][tid] = agg;
            agg += c;
        }
    }
    // Exclusive scan of the digit totals (threads >= kRadix contribute 0).
    const u32 inc = wave_inclusive_scan(agg);
    if (lane == 63) sh.wave[w] = inc;
    __syncthreads();
    if (tid < kRadix) {
        u32 off = 0;
#pragma unroll
        for (int i = 0; i < kLocalWaves; ++i)
            if (i < w) off += sh.wave[i];
        sh.start[tid] = off + inc - agg;
    }
    __syncthreads();
    // A record is a 32-bit key above a 16-bit slot (bits 16..47; all-ones
    // records read back as 48 one bits, still behind every real record): it
    // moves in two exchanges, which keeps the buffer at 4 bytes a record.
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 d = (u32)(rec[j] >> shift) & (kRadix - 1);
        rank[j] += sh.start[d] + sh.count[w][d];
        sh.exch[rank[j]] = (u32)(rec[j] >> 16);
    }
    __syncthreads();
    u32 hi[kLocalItems];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) hi[j] = sh.exch[local_slot(j)];
    __syncthreads();
    uint16_t* exch16 = reinterpret_cast<uint16_t*>(sh.exch);
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) exch16[rank[j]] = (uint16_t)rec[j];
    __syncthreads();
    // The next pass's first barrier orders these reads before its writes.
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) rec[j] = ((u64)hi[j] << 16) | exch16[local_slot(j)];
}

// Stable sort of the records by bits [lo, lo + 8*bytes), skipping bytes on
// which every valid record agrees.
__device__ void local_sort(u64 (&rec)[kLocalItems], int lo, int bytes, u32 nc, LocalShared& sh) {
    const u64 vary = local_varying_bits(rec, nc, sh);
    for (int b = 0; b < bytes; ++b) {
        const int shift = lo + 8 * b;
        if ((vary >> shift) & (kRadix - 1)) local_pass(rec, shift, sh);
    }
}

struct SubtreeArgs {
    const float* pts;
    i64 n;
    int k;
    int l0;                 // level of the subtree roots
    Geometry geo;
    const u32* sorted;      // point indices in the sorted order of round l0-1 (l0 > 0)
    int index_bytes;        // bytes of a point index that can differ
    u32* stage;             // (k+1) x n words: index, then coordinate columns; the
                            // subtree owns [first, first + |S(c)|) of each
    int32_t* perm;
    float* tree;
};

// order[q] = slot (index rank) of the q-th point of the subtree by
// (coordinate dim, original index): stable sort by the coordinate key,
// starting from index order.
__device__ void local_order(const u32* __restrict__ col, u32 nc, uint16_t* order,
                            LocalShared& sh) {
    u64 rec[kLocalItems];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const int e = local_slot(j);
        rec[j] = ~0ull;
        if ((u32)e < nc) rec[j] = ((u64)float_key(col[e]) << 16) | (u32)e;
    }
    local_sort(rec, 16, kKeyBytes, nc, sh);
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const int q = local_slot(j);
        if ((u32)q < nc) order[q] = (uint16_t)(rec[j] & 0xffff);
    }
    __syncthreads();
}

// Round t sorts every segment's points by (tag, coordinate, index) and
// moves each point to the child its sorted position falls in. Segment s
// starts at a closed-form position, so a point's sorted position is that
// start plus its rank among the points of s earlier in the (coordinate,
// index) order; that rank is all the round needs, and no record has to
// move. It is counted per wave over the 2^t live segments (ballot match on
// s - F(t)), then prefixed across waves. Count is the counter type: a
// segment on local level t of a subtree of at most kLocalMax points holds at
// most 2^(levels-t) - 1 points, so 8-bit counters would suffice wherever
// 16-bit ones no longer fit the exchange buffer (with 4096-point subtrees
// 16-bit ones always fit).
template <typename Count>
__device__ void local_round(const uint16_t* order, u32 nc, int t, const Geometry& lg,
                            LocalShared& sh) {
    Count* seg_count = reinterpret_cast<Count*>(sh.exch);  // [kLocalWaves][2^t]
    const u32 fl = (u32)full_nodes(t);
    const int segs = 1 << t;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int i = threadIdx.x; i < kLocalWaves * segs; i += kLocalBlock) seg_count[i] = 0;
    __syncthreads();
    const u64 below = (1ull << lane) - 1;
    u32 seg[kLocalItems], rank[kLocalItems];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 q = (u32)local_slot(j);
        u32 st = fl;  // fixed points (tags < F(t)) are not ranked
        if (q < nc) st = sh.tag[order[q]];
        const bool live = st >= fl && q < nc;
        const u32 b = live ? st - fl : 0;
        seg[j] = st;
        u32 miss_lo = 0, miss_hi = 0;
        for (int bit = 0; bit < t; ++bit) {
            const u64 vote = __ballot((b >> bit) & 1);
            const u32 m = (u32)((int)(b << (31 - bit)) >> 31);
            miss_lo |= (u32)vote ^ m;
            miss_hi |= (u32)(vote >> 32) ^ m;
        }
        const u64 peers = __ballot(live) & ~(((u64)miss_hi << 32) | miss_lo);
        const u32 before = __popcll(peers & below);
        u32 seen = 0;
        if (live) seen = seg_count[w * segs + b];
        rank[j] = seen + before;
        if (live && before == 0) seg_count[w * segs + b] = (Count)(seen + __popcll(peers));
    }
    __syncthreads();
    for (int b = threadIdx.x; b < segs; b += kLocalBlock) {
        u32 run = 0;
        for (int v = 0; v < kLocalWaves; ++v) {
            const u32 c = seg_count[v * segs + b];
            seg_count[v * segs + b] = (Count)run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 q = (u32)local_slot(j);
        const u64 s = seg[j];
        if (q >= nc || s < fl) continue;
        const u64 p = segment_begin(lg, s, t) + seg_count[w * segs + (s - fl)] + rank[j];
        const u64 pivot = segment_begin(lg, s, t) + subtree_size(lg, 2 * s + 1);
        sh.tag[order[q]] = (uint16_t)(p < pivot ? 2 * s + 1 : (p > pivot ? 2 * s + 2 : s));
    }
    __syncthreads();
}

__global__ __launch_bounds__(kLocalBlock, 4) void k_subtree(SubtreeArgs a) {
    __shared__ LocalShared sh;

    const u64 c = full_nodes(a.l0) + blockIdx.x;  // subtree root (global node id)
    const u32 nc = (u32)subtree_size(a.geo, c);
    if (nc == 0) return;
    u64 first = 0;  // where the subtree's points start in round l0-1's sorted order
    if (a.l0 > 0) {
        const u64 parent = (c - 1) / 2;
        const u64 seg = segment_begin(a.geo, parent, a.l0 - 1);
        const u64 pivot = seg + subtree_size(a.geo, 2 * parent + 1);
        first = (c == 2 * parent + 1) ? seg : pivot + 1;
    }

    // Order the subtree's points by original index: slot e = index rank.
    u64 rec[kLocalItems];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const int q = local_slot(j);
        rec[j] = ~0ull;
        if ((u32)q < nc) {
            const u32 i = a.sorted ? a.sorted[first + q] : (u32)q;
            rec[j] = ((u64)i << 16) | (u32)q;
        }
    }
    if (a.sorted) local_sort(rec, 16, a.index_bytes, nc, sh);
    // Stage the subtree's points once, by index rank: their indices and their
    // coordinate columns (each row of `points` is read exactly once here).
    u32* stage_idx = a.stage + first;
    if (a.k <= kRowRegs) {
        // Row loads are issued kRowBatch items at a time, before their stores.
#pragma unroll
        for (int j0 = 0; j0 < kLocalItems; j0 += kRowBatch) {
            u32 row[kRowBatch][kRowRegs];
#pragma unroll
            for (int j = 0; j < kRowBatch; ++j) {
                const u32 i = (u32)(rec[j0 + j] >> 16);
                const bool ok = (u32)local_slot(j0 + j) < nc;
#pragma unroll
                for (int d = 0; d < kRowRegs; ++d)
                    row[j][d] = ok && d < a.k ? __float_as_uint(a.pts[(i64)i * a.k + d]) : 0u;
            }
#pragma unroll
            for (int j = 0; j < kRowBatch; ++j) {
                const int e = local_slot(j0 + j);
                if ((u32)e >= nc) continue;
                stage_idx[e] = (u32)(rec[j0 + j] >> 16);
#pragma unroll
                for (int d = 0; d < kRowRegs; ++d)
                    if (d < a.k) a.stage[(u64)(d + 1) * a.n + first + e] = row[j][d];
                sh.tag[e] = 0;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const int e = local_slot(j);
            if ((u32)e >= nc) continue;
            const u32 i = (u32)(rec[j] >> 16);
            stage_idx[e] = i;
            const float* row = a.pts + (i64)i * a.k;
            for (int d = 0; d < a.k; ++d)
                a.stage[(u64)(d + 1) * a.n + first + e] = __float_as_uint(row[d]);
            sh.tag[e] = 0;
        }
    }
    auto column = [&](int d) { return a.stage + (u64)(d + 1) * a.n + first; };

    const Geometry lg = make_geometry((i64)nc);
    const int rounds = lg.levels - 1;
    const bool cached = a.k <= kCachedDims;
    // The points arrived in round l0-1's sorted order, i.e. ordered by
    // (coordinate (l0-1) mod k, index): that is already the subtree's order
    // for that dimension (slot of the arrival position q = rec's low bits).
    const int arrived_dim = a.sorted ? (a.l0 - 1) % a.k : -1;
    uint16_t* arrived = a.sorted ? sh.order[cached ? a.k - 1 : 1] : nullptr;
    if (arrived) {
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const int e = local_slot(j);
            if ((u32)e < nc) arrived[rec[j] & 0xffff] = (uint16_t)e;
        }
    }
    if (cached)
        for (int u = 0; u < a.k && u < rounds; ++u)
            if ((a.l0 + u) % a.k != arrived_dim)
                local_order(column((a.l0 + u) % a.k), nc, sh.order[u], sh);
    __syncthreads();

    for (int t = 0; t < rounds; ++t) {
        uint16_t* order = sh.order[cached ? t % a.k : 0];
        if (!cached) {
            if ((a.l0 + t) % a.k == arrived_dim) order = arrived;
            else local_order(column((a.l0 + t) % a.k), nc, order, sh);
        }
        // Counters live in the exchange buffer: 16-bit while they fit, else
        // 8-bit (then segments hold at most 3 points, see below).
        if ((size_t)kLocalWaves * ((size_t)2 << t) <= sizeof(sh.exch))
            local_round<uint16_t>(order, nc, t, lg, sh);
        else
            local_round<uint8_t>(order, nc, t, lg, sh);
    }

    // Level-order output of the subtree, in node order: the nodes of each
    // local level are one contiguous range of global ids, so the writes of
    // consecutive threads are contiguous.
    uint16_t* slot_of = sh.order[0];  // the orders are no longer needed
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const int e = local_slot(j);
        if ((u32)e < nc) slot_of[sh.tag[e]] = (uint16_t)e;
    }
    __syncthreads();
    for (u32 node = threadIdx.x; node < nc; node += kLocalBlock) {
        const u32 e = slot_of[node];
        const int lvl = level_of(node);
        const u64 g = ((c + 1) << lvl) - 1 + (node - full_nodes(lvl));
        if (g >= (u64)a.n) continue;  // cannot happen: local nodes map inside the tree
        a.perm[g] = (int32_t)stage_idx[e];
        if (!a.tree) continue;
        if (a.k <= kRowRegs) {
            u32 row[kRowRegs];
#pragma unroll
            for (int d = 0; d < kRowRegs; ++d)
                row[d] = d < a.k ? a.stage[(u64)(d + 1) * a.n + first + e] : 0u;
#pragma unroll
            for (int d = 0; d < kRowRegs; ++d)
                if (d < a.k) a.tree[(i64)g * a.k + d] = __uint_as_float(row[d]);
        } else {
            for (int d = 0; d < a.k; ++d)
                a.tree[(i64)g * a.k + d] = __uint_as_float(a.stage[(u64)(d + 1) * a.n + first + e]);
        }
    }
}

// A single point is the whole tree (no workspace is needed for N = 1).
__global__ void k_single(const float* __restrict__ pts, int k, int32_t* __restrict__ perm,
                         float* __restrict__ tree) {
    if (threadIdx.x == 0) perm[0] = 0;
    if (tree)
        for (int d = threadIdx.x; d < k; d += blockDim.x) tree[d] = pts[d];
}

// Nodes above level l0: the F(l0-1) nodes fixed before round l0-1 sit at
// their own id in that round's sorted order, and each node s on level l0-1
// is its segment's pivot.
__global__ __launch_bounds__(kBlock) void k_place_top(const float* __restrict__ pts, int k,
                                                      Geometry geo, int l0,
                                                      const u32* __restrict__ sorted,
                                                      int32_t* __restrict__ perm,
                                                      float* __restrict__ tree) {
    const u64 s = (u64)blockIdx.x * kBlock + threadIdx.x;
    if (s >= full_nodes(l0)) return;
    u64 p = s;
    if (s >= full_nodes(l0 - 1))
        p = segment_begin(geo, s, l0 - 1) + subtree_size(geo, 2 * s + 1);
    if (p >= (u64)geo.n) return;
    const u32 i = sorted[p];
    perm[s] = (int32_t)i;
    if (tree)
        for (int d = 0; d < k; ++d) tree[(i64)s * k + d] = pts[(i64)i * k + d];
}

__global__ __launch_bounds__(kBlock) void k_copy_tags(const u32* __restrict__ tag, i64 n,
                                                      u32* __restrict__ out) {
    const i64 stride = (i64)gridDim.x * kBlock;
    for (i64 e = (i64)blockIdx.x * kBlock + threadIdx.x; e < n; e += stride)
        out[e] = tag ? tag[e] : 0u;
}

// ------------------------------------------------------------ host driver

inline size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
    int kcols;          // split dimensions the global rounds can use
    i64 tiles, chunks;
    size_t cols, orders, ranks, next, tagq, keys0, keys1, vals0, vals1, extra0, extra1, totals,
        slots, chunk_slots, stage, total;
};

bool make_layout(i64 n, int k, Layout* out) {
    if (n < 0 || n > INT32_MAX || k < 1 || k > 65535) return false;
    Layout lay{};
    if (n <= 1) {
        *out = lay;
        return true;
    }
    const int levels = make_geometry(n).levels;
    // dimensions the global rounds touch: the split dimensions of rounds
    // 0 .. L-2 plus the one whose order the last written tags are kept in
    lay.kcols = levels < k ? levels : k;
    lay.tiles = (n + kTile - 1) / kTile;
    lay.chunks = (lay.tiles + kChunkTiles - 1) / kChunkTiles;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    lay.cols = take((size_t)lay.kcols * n * sizeof(float));
    lay.orders = take((size_t)lay.kcols * n * sizeof(u32));
    lay.ranks = take((size_t)lay.kcols * n * sizeof(u32));
    lay.next = take((size_t)lay.kcols * n * sizeof(u32));
    lay.tagq = take((size_t)lay.kcols * n * sizeof(u32));
    lay.keys0 = take((size_t)n * sizeof(u32));
    lay.keys1 = take((size_t)n * sizeof(u32));
    lay.vals0 = take((size_t)n * sizeof(u32));
    lay.vals1 = take((size_t)n * sizeof(u32));
    lay.extra0 = take((size_t)n * sizeof(u32));
    lay.extra1 = take((size_t)n * sizeof(u32));
    lay.totals = take((size_t)kRadix * sizeof(u32));
    lay.slots = take((size_t)lay.tiles * kRadix * sizeof(u32));
    lay.chunk_slots = take((size_t)lay.chunks * kRadix * sizeof(u32));
    lay.stage = take((size_t)(k + 1) * n * sizeof(u32));
    lay.total = off;
    *out = lay;
    return true;
}

inline int grid_for(i64 work, int per_block, int cap) {
    i64 g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (int)g;
}

bool ranges_overlap(const void* a, size_t an, const void* b, size_t bn) {
    if (!a || !b || an == 0 || bn == 0) return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

// Optional per-kernel timing: an event pair around every launch, grouped
// by kernel (names as the profiler prints them) with each launch's
// algorithmic bytes: every array the kernel must read or write, once.
struct Profiler {
    struct Rec {
        int kind;
        double bytes;
        hipEvent_t start, stop;
    };
    Rec recs[2048];
    int count = 0;
    const char* names[KDT_PROFILE_MAX_KINDS];
    int kinds = 0;
    bool failed = false;
    hipStream_t stream;

    int kind_of(const char* name) {
        for (int i = 0; i < kinds; ++i)
            if (names[i] == name) return i;
        if (kinds == KDT_PROFILE_MAX_KINDS) return -1;
        names[kinds] = name;
        return kinds++;
    }
    void begin(const char* name, double bytes) {
        const int kind = kind_of(name);
        if (count >= 2048 || kind < 0) { failed = true; return; }
        Rec& r = recs[count];
        r.kind = kind;
        r.bytes = bytes;
        if (hipEventCreate(&r.start) != hipSuccess) { failed = true; return; }
        if (hipEventCreate(&r.stop) != hipSuccess) {
            (void)hipEventDestroy(r.start);
            failed = true;
            return;
        }
        if (hipEventRecord(r.start, stream) != hipSuccess) failed = true;
    }
    void end() {
        if (failed) return;
        if (hipEventRecord(recs[count].stop, stream) != hipSuccess) failed = true;
        ++count;
    }
};

struct Timer {  // no-op unless a Profiler is attached
    Profiler* p;
    void begin(const char* name, double bytes) { if (p) p->begin(name, bytes); }
    void end() { if (p) p->end(); }
};

// Launches the three kernels of one radix pass.
struct PassLauncher {
    const Layout& lay;
    u32* tile_counts;
    u32* chunk_slots;
    hipStream_t stream;
    Timer timer;

    template <int kSrc, int kSink, bool kTags = false>
    void run(PassArgs a) {
        a.tile_counts = tile_counts;
        a.chunk_slots = chunk_slots;
        // this pass's records (at most the layout's n)
        const i64 tiles64 = (a.n + kTile - 1) / kTile;
        const unsigned tiles = (unsigned)tiles64;
        const unsigned chunks = (unsigned)((tiles64 + kChunkTiles - 1) / kChunkTiles);
        const double n = (double)a.n;
        static const char* const count_names[2] = {"k_tile_count<0>", "k_tile_count<1>"};
        // [kSrc][kSink][extra][kTags], as the profiler prints the kernels
        static const char* const scatter_names[2][3][2][2] = {
            {{{"k_tile_scatter<0, 0, false, false>", "k_tile_scatter<0, 0, false, true>"},
              {"k_tile_scatter<0, 0, true, false>", "k_tile_scatter<0, 0, true, true>"}},
             {{"k_tile_scatter<0, 1, false, false>", "k_tile_scatter<0, 1, false, true>"},
              {"k_tile_scatter<0, 1, true, false>", "k_tile_scatter<0, 1, true, true>"}},
             {{"k_tile_scatter<0, 2, false, false>", "k_tile_scatter<0, 2, false, true>"},
              {"k_tile_scatter<0, 2, true, false>", "k_tile_scatter<0, 2, true, true>"}}},
            {{{"k_tile_scatter<1, 0, false, false>", "k_tile_scatter<1, 0, false, true>"},
              {"k_tile_scatter<1, 0, true, false>", "k_tile_scatter<1, 0, true, true>"}},
             {{"k_tile_scatter<1, 1, false, false>", "k_tile_scatter<1, 1, false, true>"},
              {"k_tile_scatter<1, 1, true, false>", "k_tile_scatter<1, 1, true, true>"}},
             {{"k_tile_scatter<1, 2, false, false>", "k_tile_scatter<1, 2, false, true>"},
              {"k_tile_scatter<1, 2, true, false>", "k_tile_scatter<1, 2, true, true>"}}}};
        const bool extra = a.extra_in != nullptr;
        timer.begin(count_names[kSrc], n * 4);  // keys (or the column)
        k_tile_count<kSrc><<<chunks, kCountBlock, 0, stream>>>(a);
        timer.end();
        timer.begin("k_tile_scan", (double)chunks * kRadix * 8);
        k_tile_scan<<<kRadix, kBlock, 0, stream>>>(chunk_slots, chunks, a.digit_totals);
        timer.end();
        // in: column (4) or key+val (8); out: key+val (8) or one word (4)
        const double in = (kSrc == kSrcColumn ? 4 : 8) + (extra ? 4 : 0);
        const double out = (kSink == kSinkArrays ? 8 : 4) + (extra ? 4 : 0) + (a.rank_out ? 4 : 0);
        timer.begin(scatter_names[kSrc][kSink][extra][kTags], n * (in + out));
        if (extra)
            k_tile_scatter<kSrc, kSink, true, kTags><<<tiles, kBlock, 0, stream>>>(a);
        else
            k_tile_scatter<kSrc, kSink, false, kTags><<<tiles, kBlock, 0, stream>>>(a);
        timer.end();
    }
};

// Runs rounds 0 .. rounds-1 on the whole point set. With keep_sorted the
// last round writes its sorted order (point indices, returned in
// *sorted_out) instead of updating the tags. Otherwise the tags after
// `rounds` rounds are left in tagq of dimension rounds mod k, in that
// dimension's (coordinate, index) order, which *tags_dim returns.
kdt_status run_rounds(const float* pts, i64 n, int k, int rounds, char* ws, const Layout& lay,
                      hipStream_t stream, Timer timer, bool keep_sorted,
                      const u32** sorted_out, int* tags_dim) {
    const Geometry geo = make_geometry(n);
    const int writes = keep_sorted ? rounds - 1 : rounds;  // rounds that write tags
    // dimensions touched: split dimensions of rounds 0 .. rounds-1 and the
    // one each written round hands its tags to
    const int span = writes + 1 > rounds ? writes + 1 : rounds;
    const int kc = span < k ? span : k;
    float* cols = (float*)(ws + lay.cols);
    u32* totals = (u32*)(ws + lay.totals);
    u32* keys[2] = {(u32*)(ws + lay.keys0), (u32*)(ws + lay.keys1)};
    u32* vals[2] = {(u32*)(ws + lay.vals0), (u32*)(ws + lay.vals1)};
    auto order = [&](int d) { return (u32*)(ws + lay.orders) + (size_t)d * n; };
    auto rank = [&](int d) { return (u32*)(ws + lay.ranks) + (size_t)d * n; };
    auto next = [&](int d) { return (u32*)(ws + lay.next) + (size_t)d * n; };
    auto tagq = [&](int d) { return (u32*)(ws + lay.tagq) + (size_t)d * n; };
    PassLauncher pass{lay, (u32*)(ws + lay.slots), (u32*)(ws + lay.chunk_slots), stream, timer};
    const double N = (double)n;
    const int grid = grid_for(n, kBlock, 1 << 30);  // one element per thread: more writes in flight

    timer.begin("k_init", N * kc * 8);
    k_init<<<grid, kBlock, 0, stream>>>(pts, n, k, kc, cols);
    timer.end();

    // next_d maps the r-th point of order_d to its position in order_(d+1):
    // round l's new tags go straight to where round l+1 reads them. For
    // d >= 1 the presort of d carries rank_(d+1) (a point's position in
    // order_(d+1), in index order) as a second payload, so its sorted output
    // is next_d; the dimensions are presorted as 0, kc-1, ..., 1 so that
    // rank_(d+1) exists by then. next_0 comes from two scattered ranks.
    const int knext = writes < k ? writes : k;  // next_d needed for d < knext
    u32* extra[2] = {(u32*)(ws + lay.extra0), (u32*)(ws + lay.extra1)};
    for (int step = 0; step < kc; ++step) {
        const int d = step == 0 ? 0 : kc - step;
        const float* col = cols + (size_t)d * n;
        const bool carry = d >= 1 && d < knext;
        // Presort: order_d = point indices by (coordinate d, index). Pass p
        // reads buffer (p+1)&1 and writes buffer p&1; the last writes order_d.
        for (int p = 0; p < kKeyBytes; ++p) {
            PassArgs a{};
            a.n = n;
            a.n_all = n;
            a.shift = 8 * p;
            a.col = col;
            a.keys_in = keys[(p + 1) & 1];
            a.vals_in = vals[(p + 1) & 1];
            a.keys_out = keys[p & 1];
            a.vals_out = p == kKeyBytes - 1 ? order(d) : vals[p & 1];
            if (carry) {
                a.extra_in = p == 0 ? rank((d + 1) % k) : extra[(p + 1) & 1];
                a.extra_out = p == kKeyBytes - 1 ? next(d) : extra[p & 1];
            }
            if (p == kKeyBytes - 1 && knext > 0) a.rank_out = rank(d);
            a.digit_totals = totals;
            if (p == 0)
                pass.run<kSrcColumn, kSinkArrays>(a);
            else if (p < kKeyBytes - 1)
                pass.run<kSrcArrays, kSinkArrays>(a);
            else
                pass.run<kSrcArrays, kSinkVals>(a);
        }
    }
    if (knext > 0) {
        timer.begin("k_cross", N * 12);
        k_cross<<<grid, kBlock, 0, stream>>>(rank(0), rank(1 % k), n, next(0));
        timer.end();
    }

    // Round 0: all tags are 0.
    if (writes == 0) {
        *sorted_out = order(0);  // keep_sorted with a single round
    } else {
        timer.begin("k_round0", N * 8);
        k_round0<<<grid, kBlock, 0, stream>>>(next(0), geo, tagq(1 % k));
        timer.end();
    }

    // Round l: stable sort of the records (tag, next_d[r]) -- or (tag, point
    // index) in the final round -- kept in order_d order, by tag, one pass
    // per byte of the live tags' offset from F(l); pass p reads buffer p&1
    // and writes buffer (p+1)&1. The F(l) fixed records are not sorted: the
    // first pass writes them straight to where they end up (their tag for
    // the next round, or their node's slot of the sorted order), and later
    // passes see only the N - F(l) live records.
    for (int l = 1; l < rounds; ++l) {
        const int d = l % k;
        const int passes = tag_passes(l);
        const bool final = keep_sorted && l == rounds - 1;
        const u32 fl = (u32)full_nodes(l);
        u32* sorted = vals[passes & 1];  // final round: the whole sorted order
        for (int p = 0; p < passes; ++p) {
            PassArgs a{};
            a.n = p == 0 ? n : n - (i64)fl;
            a.n_all = n;
            a.shift = 8 * p;
            a.key_base = fl;
            a.digit_totals = totals;
            a.geo = geo;
            a.round = l;
            a.keys_in = p == 0 ? tagq(d) : keys[p & 1];
            a.vals_in = p == 0 ? (final ? order(d) : next(d)) : vals[p & 1];
            a.keys_out = keys[(p + 1) & 1];
            a.vals_out = vals[(p + 1) & 1];
            a.tag_out = tagq((l + 1) % k);
            if (final) a.fixed_vals = sorted;
            else a.fixed_tags = a.tag_out;
            const bool last = p == passes - 1;
            if (!last) {
                pass.run<kSrcArrays, kSinkArrays, true>(a);
            } else if (final) {
                a.vals_out = sorted + fl;  // live records follow the F(l) fixed ones
                *sorted_out = sorted;
                pass.run<kSrcArrays, kSinkVals, true>(a);
            } else {
                pass.run<kSrcArrays, kSinkTags, true>(a);
            }
        }
    }
    if (tags_dim) *tags_dim = rounds % k;
    return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
}

kdt_status validate(const float* pts, i64 n, int k, const void* out0, size_t out0_bytes,
                    const void* out1, size_t out1_bytes, void* ws, size_t ws_bytes,
                    Layout* lay) {
    if (!make_layout(n, k, lay)) return KDT_ERR_INVALID_ARG;
    if (n == 0) return KDT_OK;
    if (!pts || !out0) return KDT_ERR_INVALID_ARG;
    const size_t pts_bytes = (size_t)n * k * sizeof(float);
    if (ranges_overlap(pts, pts_bytes, out0, out0_bytes) ||
        ranges_overlap(pts, pts_bytes, out1, out1_bytes) ||
        ranges_overlap(out0, out0_bytes, out1, out1_bytes))
        return KDT_ERR_INVALID_ARG;
    if (lay->total > 0) {
        if (!ws || ws_bytes < lay->total || ((uintptr_t)ws & 255)) return KDT_ERR_WORKSPACE;
        if (ranges_overlap(ws, lay->total, pts, pts_bytes) ||
            ranges_overlap(ws, lay->total, out0, out0_bytes) ||
            ranges_overlap(ws, lay->total, out1, out1_bytes))
            return KDT_ERR_INVALID_ARG;
    }
    return KDT_OK;
}

// First level whose subtrees all fit one workgroup (the leftmost subtree of
// a level is the largest one).
int split_level(const Geometry& g) {
    int l = 0;
    while (subtree_size(g, full_nodes(l)) > (u64)kLocalMax) ++l;
    return l;
}

kdt_status build_impl(const float* points, int64_t N, int32_t k, int32_t* perm_out,
                      float* tree_out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream, Timer timer) {
    Layout lay;
    const size_t perm_bytes = (size_t)(N > 0 ? N : 0) * sizeof(int32_t);
    const size_t tree_bytes = tree_out ? (size_t)(N > 0 ? N : 0) * (k > 0 ? k : 0) * sizeof(float) : 0;
    kdt_status st = validate(points, N, k, perm_out, perm_bytes, tree_out, tree_bytes, workspace,
                             workspace_bytes, &lay);
    if (st != KDT_OK || N == 0) return st;
    if (N == 1) {
        timer.begin("k_single", 4.0 + (tree_out ? 8.0 * k : 0));
        k_single<<<1, 64, 0, stream>>>(points, k, perm_out, tree_out);
        timer.end();
        return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
    }
    const Geometry geo = make_geometry(N);
    const int l0 = split_level(geo);
    const u32* sorted = nullptr;
    if (l0 > 0) {
        // Global rounds 0 .. l0-1; the last one leaves its sorted order.
        st = run_rounds(points, N, k, l0, (char*)workspace, lay, stream, timer, true, &sorted,
                        nullptr);
        if (st != KDT_OK) return st;
        const u64 top = full_nodes(l0);
        timer.begin("k_place_top", (double)top * (4 + 4 + (tree_out ? 8.0 * k : 0)));
        k_place_top<<<(unsigned)((top + kBlock - 1) / kBlock), kBlock, 0, stream>>>(
            points, k, geo, l0, sorted, perm_out, tree_out);
        timer.end();
    }
    SubtreeArgs sa{};
    sa.pts = points;
    sa.n = N;
    sa.k = k;
    sa.l0 = l0;
    sa.geo = geo;
    sa.sorted = sorted;
    int bits = 0;
    for (u64 v = (u64)(N - 1); v; v >>= 1) ++bits;
    sa.index_bytes = (bits + kRadixBits - 1) / kRadixBits;
    sa.stage = (u32*)((char*)workspace + lay.stage);
    sa.perm = perm_out;
    sa.tree = tree_out;
    const i64 below = N - (i64)full_nodes(l0);  // points in the level-l0 subtrees
    // indices in (when l0 > 0), one row gathered, index + row staged and read
    // back, perm and tree out
    const double row = 4.0 * k;
    timer.begin("k_subtree", (double)below * ((l0 > 0 ? 4 : 0) + row + 2 * (4 + row) + 4 +
                                             (tree_out ? row : 0)));
    k_subtree<<<(unsigned)(1ull << l0), kLocalBlock, 0, stream>>>(sa);
    timer.end();
    return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
}

}  // namespace

extern "C" {

size_t kdt_workspace_size(int64_t N, int32_t k) {
    Layout lay;
    if (!make_layout(N, k, &lay)) return 0;
    return lay.total;
}

kdt_status kdt_build(const float* points, int64_t N, int32_t k, int32_t* perm_out,
                     float* tree_out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    return build_impl(points, N, k, perm_out, tree_out, workspace, workspace_bytes, stream,
                      Timer{nullptr});
}

kdt_status kdt_build_profiled(const float* points, int64_t N, int32_t k, int32_t* perm_out,
                              float* tree_out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, kdt_profile* profile) {
    if (!profile) return KDT_ERR_INVALID_ARG;
    Profiler* prof = new Profiler();
    prof->stream = stream;
    kdt_status st = build_impl(points, N, k, perm_out, tree_out, workspace, workspace_bytes,
                               stream, Timer{prof});
    if (hipStreamSynchronize(stream) != hipSuccess && st == KDT_OK) st = KDT_ERR_HIP;
    *profile = kdt_profile{};
    profile->kinds = prof->kinds;
    for (int i = 0; i < prof->kinds; ++i)
        for (int c = 0; prof->names[i][c] && c < KDT_PROFILE_NAME_LEN - 1; ++c)
            profile->name[i][c] = prof->names[i][c];
    for (int i = 0; i < prof->count; ++i) {
        Profiler::Rec& r = prof->recs[i];
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess && st == KDT_OK)
            st = KDT_ERR_HIP;
        profile->ms[r.kind] += ms;
        profile->launches[r.kind] += 1;
        profile->bytes[r.kind] += r.bytes;
    }
    for (int i = 0; i < prof->count; ++i) {
        (void)hipEventDestroy(prof->recs[i].start);
        (void)hipEventDestroy(prof->recs[i].stop);
    }
    if (prof->failed && st == KDT_OK) st = KDT_ERR_HIP;  // event API failure or > 32 kernels
    delete prof;
    return st;
}

kdt_status kdt_debug_tags(const float* points, int64_t N, int32_t k, int32_t rounds,
                          uint32_t* tags_out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    Layout lay;
    const size_t tag_bytes = (size_t)(N > 0 ? N : 0) * sizeof(u32);
    kdt_status st = validate(points, N, k, tags_out, tag_bytes, nullptr, 0, workspace,
                             workspace_bytes, &lay);
    if (st != KDT_OK || N == 0) return st;
    const int max_rounds = make_geometry(N).levels - 1;
    if (rounds < 0 || rounds > max_rounds) return KDT_ERR_INVALID_ARG;
    if (rounds == 0) {
        k_copy_tags<<<grid_for(N, kBlock * 4, 8192), kBlock, 0, stream>>>(nullptr, N, tags_out);
        return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
    }
    int d = 0;
    st = run_rounds(points, N, k, rounds, (char*)workspace, lay, stream, Timer{nullptr}, false,
                    nullptr, &d);
    if (st != KDT_OK) return st;
    const u32* tagq = (const u32*)((char*)workspace + lay.tagq) + (size_t)d * N;
    const u32* order = (const u32*)((char*)workspace + lay.orders) + (size_t)d * N;
    k_unpermute<<<grid_for(N, kBlock * 4, 8192), kBlock, 0, stream>>>(tagq, order, N, tags_out);
    return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
}

int64_t kdt_closed_subtree_size(int64_t N, int64_t s) {
    if (N <= 0 || N > INT32_MAX || s < 0) return 0;
    if (s >= N) return 0;
    return (int64_t)subtree_size(make_geometry(N), (u64)s);
}

int64_t kdt_closed_segment_begin(int64_t N, int64_t s, int32_t l) {
    if (N <= 0 || N > INT32_MAX || s < 0 || s >= N) return -1;
    const Geometry g = make_geometry(N);
    if (l < 0 || l >= g.levels || level_of((u64)s) != l) return -1;
    return (int64_t)segment_begin(g, (u64)s, l);
}

int32_t kdt_round_passes(int64_t N, int32_t l) {
    if (N <= 1 || N > INT32_MAX) return -1;
    if (l < 0 || l >= make_geometry(N).levels - 1) return -1;
    return l == 0 ? 0 : tag_passes(l);
}

const char* kdt_status_string(kdt_status status) {
    switch (status) {
        case KDT_OK: return "ok";
        case KDT_ERR_INVALID_ARG: return "invalid argument";
        case KDT_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case KDT_ERR_HIP: return "HIP kernel launch failed";
    }
    return "unknown status";
}

}  // extern "C"
