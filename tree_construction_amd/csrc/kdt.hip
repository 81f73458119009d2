// Left-balanced k-d tree build for MI355X (gfx950): the tag-based
// "trickle-down" construction of I. Wald, "GPU-friendly, Parallel, and
// (Almost-)In-Place Construction of Left-Balanced k-d Trees" (arXiv
// 2211.00120), cited as [W] with the paragraph that states each fact.
//
// Round l of [W] sorts every point by (tag, coordinate l mod k, original
// index) and refines every tag from its sorted position: in the segment of
// tag s, the point at position sb(s) + ss(2s+1) becomes node s, the points
// before it take tag 2s+1 and the points after it tag 2s+2.
//
// How the rounds are organised here:
//   * Every split dimension d has an array A_d of point records (the
//     coordinates the global rounds split on, then the original index) kept
//     in round order: sorted by (tag, coordinate d, index). When d is first
//     used all tags are still those of one level, and A_d is built by a
//     stable LSD radix sort of (key(x_d), index) from index order whose last
//     pass writes the records ("presort").
//   * A tag update only ever compares a point with the pivot of its node:
//     the point moves left iff its (coordinate, index) is below the pivot's.
//     So from the pivots (one 8-byte entry per node, a few KB) any array can
//     recompute the tags of its own points, and no per-point tag ever has to
//     move between arrays. Round l re-sorts A_(l mod k) from the tags it had
//     when last used (level l0) to level-l tags: one stable radix pass whose
//     digit is the point's path down the l - l0 levels in between, found by
//     walking the pivots. Equal digits keep their order, so each new segment
//     is still sorted by (coordinate, index): the array is in round l's sort
//     order. The records of one digit of a tile go to one contiguous run of
//     the output, so every global pass streams.
//   * The pivot of each node on level l then sits at its closed-form
//     position; it is copied to the pivot table and to the output.
//   * Once every subtree on some level holds at most 4096 points, one
//     workgroup per subtree runs the remaining rounds in LDS.
//
// A radix pass is reduce-then-scan: digit counts of each tile, a scan of
// the per-chunk counts per digit, and a scatter that ranks each tile again
// (wave64 ballots, stable multi-split) and writes it. No workgroup ever
// waits on another.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "kdt.h"

namespace {

typedef uint8_t u8;
typedef uint32_t u32;
typedef uint64_t u64;
typedef int64_t i64;
typedef u32 v4u __attribute__((ext_vector_type(4)));  // for the non-temporal builtins
typedef u32 v2u __attribute__((ext_vector_type(2)));

constexpr int kRadixBits = 8;
constexpr int kRadix = 1 << kRadixBits;
constexpr int kBlock = 256;                // threads per workgroup
constexpr int kWaves = kBlock / 64;        // wave64
constexpr int kPartItems = 8;              // records per thread in a tile
constexpr int kPartTile = kBlock * kPartItems;  // records per tile
constexpr int kKeyBytes = 4;               // order-preserving coordinate key
constexpr int kMaxDescent = kRadixBits;    // levels one re-sort pass walks
#ifndef KDT_SELECT_DEPTH
#define KDT_SELECT_DEPTH 6
#endif
constexpr int kSelectDepth = KDT_SELECT_DEPTH;  // deepest walk a split-widest round may leave to the next pass
static_assert(kSelectDepth <= kMaxDescent, "one pass per walk");
#ifndef KDT_PLAIN_DELTA
#define KDT_PLAIN_DELTA 4
#endif
constexpr int kPlainDelta = KDT_PLAIN_DELTA;  // re-sort walks from which the scatter stores plainly
constexpr int kMaxRounds = 32;             // global rounds (levels) at most
static_assert(kBlock == kRadix, "the tile kernels map one thread to one digit");

// ------------------------------------------------------------ tree geometry
// Level-order complete tree with N nodes ([W], indexing paragraph):
// level(i) = floor(log2(i+1)), numLevels(N) = level(N-1)+1, F(l) = 2^l - 1.

struct Geometry {
    i64 n;      // nodes (= points)
    int levels; // L = numLevels(N)
    i64 last;   // nodes on the last level: M = N - F(L-1)
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

// Live position of the first point of the j-th subtree on level l: its
// position in round l's sorted order counted after the F(l) points already
// fixed above level l ([W], sb/ss paragraph: sb = F(l) + this; derived).
// The j subtrees to its left hold 2^dd - 1 full-level nodes each plus the
// last-level nodes under them, min(M, j * 2^dd).
__host__ __device__ inline u64 live_begin(const Geometry& g, u64 j, int l) {
    int dd = g.levels - 1 - l;
    u64 under = j << dd;
    if (under > (u64)g.last) under = (u64)g.last;
    return j * ((1ull << dd) - 1) + under;
}

// First sorted position of subtree s (on level l) in the round that fixes
// level l: the F(l) fixed nodes sort first, then the live segments.
__host__ __device__ inline u64 segment_begin(const Geometry& g, u64 s, int l) {
    return full_nodes(l) + live_begin(g, s - full_nodes(l), l);
}

// Inverse of live_begin: the j whose segment on level l holds live position
// p. The first q = M >> dd subtrees have a full share of the last level
// (2u - 1 points, u = 2^dd), subtree q a share of r = M mod u, the rest none
// (u - 1 points).
__host__ __device__ inline u64 live_segment(const Geometry& g, u64 p, int l) {
    const int dd = g.levels - 1 - l;
    if (dd == 0) return p;  // last level: one point per segment
    const u64 u = 1ull << dd;
    const u64 q = (u64)g.last >> dd, r = (u64)g.last & (u - 1);
    const u64 full = q * (2 * u - 1);
    // positions and divisors stay below 2^32 (N < 2^31), so 32-bit division
    if (p < full) return (u32)p / (u32)(2 * u - 1);
    const u64 rest = p - full;
    if (rest < u - 1 + r) return q;
    return q + 1 + (u32)(rest - (u - 1 + r)) / (u32)(u - 1);
}

// Points of the first j0 subtrees on level l0 whose level-l1 ancestor
// (l1 = l0 + delta) is the b-th level-l1 node under their level-l0 one:
// the sizes of the level-l1 subtrees with in-level index j*2^delta + b,
// j < j0. A level-l1 subtree with in-level index i holds u - 1 full-level
// nodes plus u, r or 0 last-level ones for i < q, i == q, i > q (u = 2^dd,
// q = M >> dd, r = M mod u).
__host__ __device__ inline u64 bin_prefix(const Geometry& g, u64 j0, u32 b, int l1, int delta) {
    const int dd = g.levels - 1 - l1;
    const u64 u = 1ull << dd;
    const u64 q = (u64)g.last >> dd, r = (u64)g.last & (u - 1);
    u64 h = j0 * (u - 1);
    if (q > b) {
        const u64 c = ((q - b - 1) >> delta) + 1;  // i = j*2^delta + b < q
        h += u * (c < j0 ? c : j0);
    }
    if (q >= b && ((q - b) & ((1ull << delta) - 1)) == 0 && ((q - b) >> delta) < j0) h += r;
    return h;
}

// The same closed forms for one level in 32-bit arithmetic (every value is
// at most N < 2^31), with the level's constants precomputed: u = 2^dd,
// q = M >> dd, r = M mod u.
struct LevelShape {
    u32 dd, q, r, last;  // last = M
};

inline LevelShape level_shape(const Geometry& g, int l) {
    LevelShape s;
    s.dd = (u32)(g.levels - 1 - l);
    s.q = (u32)((u64)g.last >> s.dd);
    s.r = (u32)((u64)g.last & ((1ull << s.dd) - 1));
    s.last = (u32)g.last;
    return s;
}

__device__ inline u32 live_begin32(const LevelShape& s, u32 j) {
    const u32 under = j << s.dd;
    return j * ((1u << s.dd) - 1) + (under < s.last ? under : s.last);
}

// Size of the subtree of the node with in-level index i on the level of s.
__device__ inline u32 subtree_size32(const LevelShape& s, u32 i) {
    const u32 u = 1u << s.dd, under = i << s.dd;
    const u32 extra = s.last > under ? (s.last - under < u ? s.last - under : u) : 0u;
    return (u - 1) + extra;
}

__device__ inline u32 bin_prefix32(const LevelShape& s, u32 j0, u32 b, int delta) {
    const u32 u = 1u << s.dd;
    u32 h = j0 * (u - 1);
    if (s.q > b) {
        const u32 c = ((s.q - b - 1) >> delta) + 1;
        h += u * (c < j0 ? c : j0);
    }
    if (s.q >= b && ((s.q - b) & ((1u << delta) - 1)) == 0 && ((s.q - b) >> delta) < j0) h += s.r;
    return h;
}

// Order-preserving map of float bits to unsigned: IEEE order with -0 == +0.
// Pure bit tests, so denormals are never flushed.
__host__ __device__ inline u32 float_key(u32 b) {
    if ((b & 0x7fffffffu) == 0) return 0x80000000u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Float bits of a key: exact except that both zeros come back as +0.
__host__ __device__ inline u32 key_bits(u32 key) { return key >= 0x80000000u ? key & 0x7fffffffu : ~key; }

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

// Exclusive scan of one 64-bit value per thread across a workgroup of
// kNWaves waves (used for two 32-bit scans at once whose sums cannot carry
// out of 32 bits).
template <int kNWaves>
__device__ inline u64 block_exclusive_scan64(u64 v, u64* s_wave) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    u64 inc = wave_inclusive_scan64(v);
    if (lane == 63) s_wave[w] = inc;
    __syncthreads();
    u64 off = 0;
#pragma unroll
    for (int i = 0; i < kNWaves; ++i)
        if (i < w) off += s_wave[i];
    __syncthreads();
    return off + inc - v;
}

// One bit of the wave's digit match: ORs into miss the lanes whose bit b of
// their digit differs from this lane's. The sign-extending bit extract gives
// this lane's bit as a mask (0 or all ones) in one instruction, and the
// ballot reads the same mask.
__device__ inline void match_bit(u32 d, int b, u32& miss_lo, u32& miss_hi) {
    u32 m = (u32)__builtin_amdgcn_sbfe((int)d, b, 1);
    asm("" : "+v"(m));  // (opaque: the vote compares m, no second bit test)
    const u64 vote = __ballot(m != 0);
    // miss |= vote ^ m, one three-input bit operation per half (truth
    // table 0xF6 over (miss, vote, m), miss the most significant input)
    miss_lo = __builtin_amdgcn_bitop3_b32(miss_lo, (u32)vote, m, 0xF6);
    miss_hi = __builtin_amdgcn_bitop3_b32(miss_hi, (u32)(vote >> 32), m, 0xF6);
}

// Rank inside the wave of each of this thread's records by its digit
// (nbits bits): lanes holding the same digit are found with nbits ballots
// (a lane's peers are the lanes that never disagree with it on a bit: the OR
// over bits of vote ^ own-bit-mask, inverted), and the lowest such lane
// bumps the wave's counter for the digit. rank[j] = records of the same
// digit earlier in the wave's rows (row j of every lane precedes row j+1).
// Invalid records are neither ranked nor counted. count[] (the wave's own
// row) must be zero on entry and holds the wave's digit totals on return.
template <int kN>
__device__ inline void wave_rank(const u32 (&digit)[kN], const bool (&valid)[kN], int nbits,
                                 u32* count, u32 (&rank)[kN]) {
    const int lane = threadIdx.x & 63;
    const u64 below = (1ull << lane) - 1;
#pragma unroll
    for (int j = 0; j < kN; ++j) {
        const u32 d = digit[j];
        u32 miss_lo = 0, miss_hi = 0;
        for (int b = 0; b < nbits; ++b) match_bit(d, b, miss_lo, miss_hi);
        const u64 peers = __ballot(valid[j]) & ~(((u64)miss_hi << 32) | miss_lo);
        const u32 before = __popcll(peers & below);
        u32 seen = 0;
        if (valid[j]) seen = count[d];
        rank[j] = seen + before;
        if (valid[j] && before == 0) count[d] = seen + (u32)__popcll(peers);
    }
}

// ---------------------------------------------------- tiles of point records
// Every global pass works on tiles of kPartTile consecutive records, wave w
// owning kPartItems rows of 64 (item j of a lane is record wbase + 64 j).
// Workgroups are dealt to the 8 XCDs in turn, so tile t of workgroup b is
// chosen to give each XCD one contiguous range of tiles: the cache lines two
// neighbouring tiles both write then meet in one L2.
constexpr int kXcds = 8;

__device__ inline u32 xcd_tile(u32 tiles) {
    const u32 per = (tiles + kXcds - 1) / kXcds;
    return (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
}

inline u32 xcd_grid(u64 tiles) { return (u32)((tiles + kXcds - 1) / kXcds * kXcds); }

// The same for block b of a pass whose blocks start at a multiple of kXcds
// within a batched launch (so that b and blockIdx.x share the XCD).
__device__ inline u32 xcd_tile_of(u32 b, u32 tiles) {
    const u32 per = (tiles + kXcds - 1) / kXcds;
    return (b % kXcds) * per + b / kXcds;
}

enum Src { kSrcRows = 0, kSrcRecords = 1 };

// Where the records of a pass come from: kSrcRows builds the record of
// point e from its row of `points` (the keys of its first words-1
// coordinates, then e), in index order; kSrcRecords reads records of
// `words` words. Records carry keys, not float bits, so that every
// comparison and digit is a plain unsigned one.
// Records of at most four words are stored whole (one vector access each);
// wider records are planar: word w of every record in plane w, `plane`
// words long, so that each per-word access of a wave is one contiguous run.
constexpr int kWholeWords = 4;

__host__ __device__ inline u64 rec_word_index(int words, u64 plane, u64 e, int w) {
    return words > kWholeWords ? (u64)w * plane + e : e * (u64)words + (u64)w;
}

struct RecordSource {
    const float* pts;
    int k;
    const u32* in;
    int words;
    i64 n;
    u64 plane;  // words > kWholeWords: distance between the planes of `in`
    // planar records in index order: the index word of record e is e, not
    // read (so that the first words-1 planes of a wider copy serve)
    bool position_index;
};

template <int kSrc>
__device__ inline u32 source_word(const RecordSource& s, u64 e, int w) {
    if (kSrc == kSrcRecords) {
        if (s.position_index && w == s.words - 1) return (u32)e;
        return s.in[rec_word_index(s.words, s.plane, e, w)];
    }
    return w < s.words - 1 ? float_key(__float_as_uint(s.pts[e * s.k + w])) : (u32)e;
}

// This thread's records of a tile. kW > 0 (at most 4 words): held in
// registers, one array per word so that every index is a compile-time
// constant; kW = 0 (wider records): words are read from the source when
// needed (the tile's lines are then in L2).
template <int kSrc, int kW>
struct RecordTile {
    static_assert(kW >= 0 && kW <= 4 && kW != 1, "record width");
    u32 w0[kPartItems], w1[kPartItems], w2[kPartItems], w3[kPartItems];

    __device__ __forceinline__ void load(const RecordSource& s, i64 wbase) {
        if constexpr (kW > 0) {
#pragma unroll
            for (int j = 0; j < kPartItems; ++j) {
                const i64 e = wbase + (i64)j * 64;
                w0[j] = w1[j] = w2[j] = w3[j] = 0;
                if (e >= s.n) continue;
                if constexpr (kSrc == kSrcRows) {
                    // non-temporal like the records below: one read per pass
                    const u32* row = reinterpret_cast<const u32*>(s.pts) + (u64)e * s.k;
                    w0[j] = __builtin_nontemporal_load(row);
                    if constexpr (kW > 2) w1[j] = __builtin_nontemporal_load(row + 1);
                    if constexpr (kW > 3) w2[j] = __builtin_nontemporal_load(row + 2);
                    if constexpr (kW == 2) w1[j] = (u32)e;
                    if constexpr (kW == 3) w2[j] = (u32)e;
                    if constexpr (kW == 4) w3[j] = (u32)e;
                } else {
                    // Non-temporal: a presort pass reads each record once, and
                    // the cache is left to the partly written lines of its runs.
                    const u32* src = s.in + (u64)e * kW;
                    if constexpr (kW == 4) {
                        const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(src));
                        w0[j] = v[0];
                        w1[j] = v[1];
                        w2[j] = v[2];
                        w3[j] = v[3];
                    } else if constexpr (kW == 3) {
                        w0[j] = src[0];
                        w1[j] = src[1];
                        w2[j] = src[2];
                    } else {
                        const v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(src));
                        w0[j] = v[0];
                        w1[j] = v[1];
                    }
                }
            }
            if constexpr (kSrc == kSrcRows) {
                // keys only once every row load is in flight (inside the
                // loads' branches the first use would wait for each load)
#pragma unroll
                for (int j = 0; j < kPartItems; ++j) {
                    w0[j] = float_key(w0[j]);
                    if constexpr (kW > 2) w1[j] = float_key(w1[j]);
                    if constexpr (kW > 3) w2[j] = float_key(w2[j]);
                }
            }
        }
    }
    // The same for records (kW > 0) with no branch per item: a record past
    // the end loads the last one instead and reads as zeros, so that every
    // load is in flight before the first word is used.
    __device__ __forceinline__ void load_all(const RecordSource& s, i64 wbase) {
        static_assert(kSrc == kSrcRecords && kW > 0, "records held in registers");
#pragma unroll
        for (int j = 0; j < kPartItems; ++j) {
            const i64 e = wbase + (i64)j * 64;
            const u32* src = s.in + (u64)(e < s.n ? e : s.n - 1) * kW;
            if constexpr (kW == 4) {
                const uint4 v = *reinterpret_cast<const uint4*>(src);
                w0[j] = v.x;
                w1[j] = v.y;
                w2[j] = v.z;
                w3[j] = v.w;
            } else if constexpr (kW == 3) {
                w0[j] = src[0];
                w1[j] = src[1];
                w2[j] = src[2];
                w3[j] = 0;
            } else {
                const uint2 v = *reinterpret_cast<const uint2*>(src);
                w0[j] = v.x;
                w1[j] = v.y;
                w2[j] = w3[j] = 0;
            }
        }
#pragma unroll
        for (int j = 0; j < kPartItems; ++j) {
            if (wbase + (i64)j * 64 < s.n) continue;
            w0[j] = w1[j] = w2[j] = w3[j] = 0;
        }
    }
    // Word w of item j (record e); w is uniform across the wave. The word is
    // picked with masks, not a select, so that the compiler cannot turn the
    // choice back into an indexed (scratch) array.
    __device__ __forceinline__ u32 word(const RecordSource& s, int j, i64 e, int w) const {
        if constexpr (kW == 0) {
            return source_word<kSrc>(s, (u64)e, w);
        } else {
            const u32 m0 = w == 0 ? ~0u : 0u, m1 = w == 1 ? ~0u : 0u;
            const u32 m2 = w == 2 ? ~0u : 0u, m3 = w == 3 ? ~0u : 0u;
            u32 v = (w0[j] & m0) | (w1[j] & m1);
            if constexpr (kW > 2) v |= w2[j] & m2;
            if constexpr (kW > 3) v |= w3[j] & m3;
            return v;
        }
    }
    // Word kI of item j, chosen at compile time.
    template <int kI>
    __device__ __forceinline__ u32 at(int j) const {
        static_assert(kI >= 0 && kI < 4, "word");
        if constexpr (kI == 0) return w0[j];
        else if constexpr (kI == 1) return w1[j];
        else if constexpr (kI == 2) return w2[j];
        else return w3[j];
    }
    __device__ __forceinline__ uint4 quad(int j) const { return make_uint4(w0[j], w1[j], w2[j], w3[j]); }
    // Non-temporal stores: the output is read by a later pass, not this one,
    // and write-backs of dirty lines would otherwise land in the next pass.
    __device__ __forceinline__ void store(const RecordSource& s, u32* out, int j, i64 e, u64 pos) const {
        if constexpr (kW == 4) {
            const v4u v = {w0[j], w1[j], w2[j], w3[j]};
            __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(out + pos * 4));
        } else if constexpr (kW == 3) {
            __builtin_nontemporal_store(w0[j], out + pos * 3);
            __builtin_nontemporal_store(w1[j], out + pos * 3 + 1);
            __builtin_nontemporal_store(w2[j], out + pos * 3 + 2);
        } else if constexpr (kW == 2) {
            const v2u v = {w0[j], w1[j]};
            __builtin_nontemporal_store(v, reinterpret_cast<v2u*>(out + pos * 2));
        } else {
            copy_words(s, out, e, pos);
        }
    }
    // Wide records (kW = 0), from the source word by word: a batch of loads
    // in flight before their stores (as far as the compiler knows the
    // source and the output may alias, so a load behind a store would wait
    // for the one before it).
    __device__ __forceinline__ static void copy_words(const RecordSource& s, u32* out, i64 e, u64 pos) {
        constexpr int kBatch = 8;
        for (int w0 = 0; w0 < s.words; w0 += kBatch) {
            u32 v[kBatch];
#pragma unroll
            for (int g = 0; g < kBatch; ++g)
                if (w0 + g < s.words) v[g] = source_word<kSrc>(s, (u64)e, w0 + g);
#pragma unroll
            for (int g = 0; g < kBatch; ++g)
                if (w0 + g < s.words) out[rec_word_index(s.words, s.plane, pos, w0 + g)] = v[g];
        }
    }
    // Plain stores: where a wave's stores land in many short runs, the
    // pieces of a line meet in L2 before it is written back.
    __device__ __forceinline__ void store_plain(const RecordSource& s, u32* out, int j, i64 e, u64 pos) const {
        if constexpr (kW == 4) {
            *reinterpret_cast<uint4*>(out + pos * 4) = make_uint4(w0[j], w1[j], w2[j], w3[j]);
        } else if constexpr (kW == 3) {
            out[pos * 3] = w0[j];
            out[pos * 3 + 1] = w1[j];
            out[pos * 3 + 2] = w2[j];
        } else if constexpr (kW == 2) {
            *reinterpret_cast<uint2*>(out + pos * 2) = make_uint2(w0[j], w1[j]);
        } else {
            store(s, out, j, e, pos);
        }
    }
};

// A presort tile is larger than a re-sort tile: kSortBlock threads of
// kPartItems records, so that each of the 256 digit runs a tile writes is
// twice as long. Presort digit counts are kept per tile (tile-major rows,
// for the tiles of one chunk) and per chunk of kChunkTiles tiles
// (digit-major rows, scanned).
constexpr int kSortBlock = 512;
constexpr int kSortWaves = kSortBlock / 64;
constexpr int kSortTile = kSortBlock * kPartItems;
constexpr int kChunkTiles = 2;
constexpr int kCountBlock = kSortBlock * kChunkTiles;  // one count workgroup per chunk
static_assert(kCountBlock <= 1024, "one workgroup counts a whole chunk");
static_assert(kSortBlock >= kRadix, "a presort thread per digit");

// One workgroup per digit d: row d of `chunk` (the digit's count in each
// chunk) becomes the exclusive prefix over the chunks; totals[d] = the
// row's sum (if totals is given). Each thread scans a contiguous run of
// kScanRun chunks; longer rows loop over runs. The runs are loaded and
// stored in coalesced order and handed to their threads through LDS (rows
// of kScanRun + 1 words, so that a thread's run reads without bank
// conflicts): a thread reading its own run from memory would touch a
// different line with every lane of each load.
constexpr int kScanRun = 16;
// One workgroup of kThreads scans one row (digit) in runs of
// kThreads * kScanRun entries.
template <int kThreads>
__device__ __forceinline__ void chunk_scan_row(u32* __restrict__ row, i64 chunks, u32* __restrict__ totals, int d) {
    constexpr int kW = kThreads / 64;
    constexpr int kPitch = kScanRun + 1;
    __shared__ u32 s_wave[kW];
    __shared__ u32 s_carry;
    __shared__ u32 s_run[kThreads * kPitch];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // slot of the chunk at offset e of the stretch: thread e / kScanRun's run
    auto slot = [](int e) { return (e / kScanRun) * kPitch + e % kScanRun; };
    if (chunks <= kThreads) {  // a short row: one count a thread, no staging
        const u32 v = tid < chunks ? row[tid] : 0u;
        const u32 inc = wave_inclusive_scan(v);
        if (lane == 63) s_wave[w] = inc;
        __syncthreads();
        u32 off = inc - v, total = 0;
#pragma unroll
        for (int i = 0; i < kW; ++i) {
            off += i < w ? s_wave[i] : 0u;
            total += s_wave[i];
        }
        if (tid < chunks) row[tid] = off;
        if (totals && tid == 0) totals[d] = total;
        return;
    }
    if (tid == kThreads - 1) s_carry = 0;
    for (i64 t0 = 0; t0 < chunks; t0 += (i64)kThreads * kScanRun) {
#pragma unroll
        for (int j = 0; j < kScanRun; ++j) {
            const int e = j * kThreads + tid;
            s_run[slot(e)] = t0 + e < chunks ? row[t0 + e] : 0u;
        }
        __syncthreads();  // the runs staged; s_carry written; s_wave's last readers done
        u32 v[kScanRun], sum = 0;
#pragma unroll
        for (int i = 0; i < kScanRun; ++i) {
            v[i] = s_run[tid * kPitch + i];
            sum += v[i];
        }
        const u32 carry = s_carry;
        const u32 inc = wave_inclusive_scan(sum);
        if (lane == 63) s_wave[w] = inc;
        __syncthreads();
        u32 off = carry + inc - sum;
#pragma unroll
        for (int i = 0; i < kW; ++i)
            if (i < w) off += s_wave[i];
        // (every thread read s_carry before the barrier above)
        if (tid == kThreads - 1) s_carry = off + sum;
#pragma unroll
        for (int i = 0; i < kScanRun; ++i) {
            s_run[tid * kPitch + i] = off;  // (this thread's own run: read above)
            off += v[i];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kScanRun; ++j) {
            const int e = j * kThreads + tid;
            if (t0 + e < chunks) row[t0 + e] = s_run[slot(e)];
        }
        __syncthreads();  // the stores' LDS reads done before the next stretch's writes
    }
    __syncthreads();  // (an empty row: s_carry's first write)
    if (totals && tid == 0) totals[d] = s_carry;
}

template <int kThreads>
__device__ __forceinline__ void chunk_scan(u32* __restrict__ chunk, i64 chunks, u32* __restrict__ totals) {
    chunk_scan_row<kThreads>(chunk + (u64)blockIdx.x * chunks, chunks, totals, blockIdx.x);
}

__global__ __launch_bounds__(kBlock) void k_chunk_scan(u32* __restrict__ chunk, i64 chunks,
                                                       u32* __restrict__ totals) {
    chunk_scan<kBlock>(chunk, chunks, totals);
}
// Rows longer than kBlock counts: four times the threads, so that rows of up
// to 1024 counts take one count a thread and longer ones a quarter of the
// stretches (normal_4m_k16, whose 53 sort passes scan rows of 512 chunk
// counts: 3.43 -> 3.38 ms a build; uniform_1m_k3 0.467 -> 0.459 ms).
constexpr int kWideScanBlock = 1024;
__global__ __launch_bounds__(kWideScanBlock) void k_chunk_scan_wide(u32* __restrict__ chunk, i64 chunks,
                                                                    u32* __restrict__ totals) {
    chunk_scan<kWideScanBlock>(chunk, chunks, totals);
}

// Given each wave's digit counts hist[v][d] for the kChunkTiles tiles of a
// chunk (waves g*kWaves .. g*kWaves+kWaves-1 counted tile g), writes every
// tile's row of `bins` counts and the chunk's count of each digit.
__device__ inline void write_chunk_counts(const u32 (*hist)[kRadix], u32 (*rows)[kRadix], int bins,
                                          u32 chunk_index, u64 chunks, u64 tiles,
                                          u32* tile_counts, u32* chunk_counts) {
    const int tid = threadIdx.x, g = tid / kSortBlock, d = tid % kSortBlock;
    const u64 t = (u64)chunk_index * kChunkTiles + g;
    if (d < bins) {
        u32 total = 0;
#pragma unroll
        for (int v = 0; v < kSortWaves; ++v) total += hist[g * kSortWaves + v][d];
        if (t < tiles) tile_counts[t * bins + d] = total;
        rows[g][d] = total;
    }
    __syncthreads();
    if (tid < bins) {
        u32 sum = 0;
#pragma unroll
        for (int c = 0; c < kChunkTiles; ++c) sum += rows[c][tid];
        chunk_counts[(u64)tid * chunks + chunk_index] = sum;
    }
}

// ------------------------------------------------- presort (LSD radix sort)
// The presort of dimension d is kKeyBytes stable passes over the point
// records, each by one byte of key(x_d), least significant first, starting
// from index order (the first pass builds the records from the rows). A
// pass is three launches: k_sort_count (digit counts of each tile),
// k_chunk_scan (per digit, exclusive scan over the chunks, and the digit
// totals) and k_sort_scatter (ranks each tile again, stages it in LDS in
// sorted order and writes each digit's run contiguously). No workgroup
// ever waits on another.
struct SortArgs {
    RecordSource src;
    u32* out;           // records, words each, in this pass's order
    int dim;            // coordinate whose key is sorted
    int shift;          // digit = (key >> shift) & 255
    const u8* digits;   // this pass's digit of every record, in input order
    u8* next_digits;    // the next pass's digit of every record, in output
                        //   order (nullptr after the last pass)
    int next_dim;       // the next pass's digit: (key of next_dim >> next_shift) & 255
    int next_shift;
    u32 tiles;
    u64 chunks;
    u32* tile_counts;   // tiles x 256: digit counts of each tile
    u32* chunk_counts;  // 256 x chunks: digit counts of each chunk, then the
                        //   counts of the digit in the chunks before it
    const u32* totals;  // 256: records of each digit
};

// The first presort pass's digit (low key byte) of every point in every
// dimension the rounds use: digits0[d][e], from one read of the rows.
__global__ __launch_bounds__(kBlock) void k_first_digits(const float* __restrict__ pts, i64 n,
                                                         int k, int kr, u8* __restrict__ digits0) {
    const i64 stride = (i64)gridDim.x * kBlock;
    for (i64 e = (i64)blockIdx.x * kBlock + threadIdx.x; e < n; e += stride) {
        const u32* row = reinterpret_cast<const u32*>(pts) + (u64)e * k;
        for (int d = 0; d < kr; ++d) digits0[(u64)d * n + e] = (u8)float_key(row[d]);
    }
}

// The same for kK <= 4 coordinates and rows starting on 16 bytes: a thread
// takes four consecutive points, their rows read as kK 16-byte words, and
// writes each dimension's four digits as one word when n is a multiple of 4
// (every dimension's digits then start on a word), else as four bytes. The
// n mod 4 last points go through the per-point loop.
template <int kK>
__global__ __launch_bounds__(kBlock) void k_first_digits4(const float* __restrict__ pts, i64 n, int kr,
                                                          u8* __restrict__ digits0) {
    const i64 stride = (i64)gridDim.x * kBlock;
    const i64 quads = n / 4;
    const bool whole = n % 4 == 0;
    for (i64 q = (i64)blockIdx.x * kBlock + threadIdx.x; q < quads; q += stride) {
        const uint4* src = reinterpret_cast<const uint4*>(pts) + (u64)q * kK;
        u32 w[4 * kK];
#pragma unroll
        for (int i = 0; i < kK; ++i) {
            const uint4 v = src[i];
            w[4 * i] = v.x;
            w[4 * i + 1] = v.y;
            w[4 * i + 2] = v.z;
            w[4 * i + 3] = v.w;
        }
#pragma unroll
        for (int d = 0; d < kK; ++d) {
            if (d >= kr) break;
            u32 packed = 0;
#pragma unroll
            for (int p = 0; p < 4; ++p) packed |= (float_key(w[p * kK + d]) & 0xffu) << (8 * p);
            u8* dst = digits0 + (u64)d * n + (u64)q * 4;
            if (whole) {
                *reinterpret_cast<u32*>(dst) = packed;
            } else {
#pragma unroll
                for (int p = 0; p < 4; ++p) dst[p] = (u8)(packed >> (8 * p));
            }
        }
    }
    for (i64 e = quads * 4 + (i64)blockIdx.x * kBlock + threadIdx.x; e < n; e += stride) {
        const u32* row = reinterpret_cast<const u32*>(pts) + (u64)e * kK;
        for (int d = 0; d < kr; ++d) digits0[(u64)d * n + e] = (u8)float_key(row[d]);
    }
}

// Records wider than kWholeWords, of every point in index order, from one
// read of the rows: planar (plane d < words-1 the key of coordinate d, the
// last plane the index), with the first presort pass's digit of each
// dimension (the keys' low bytes). The presorts read their first pass from
// here instead of gathering one word of every row per staging round.
__global__ __launch_bounds__(kBlock) void k_planar_records(const float* __restrict__ pts, i64 n, int k,
                                                           int words, u32* __restrict__ out,
                                                           u8* __restrict__ digits0) {
    const i64 stride = (i64)gridDim.x * kBlock;
    for (i64 e = (i64)blockIdx.x * kBlock + threadIdx.x; e < n; e += stride) {
        const u32* row = reinterpret_cast<const u32*>(pts) + (u64)e * k;
        for (int d = 0; d < words - 1; ++d) {
            const u32 key = float_key(row[d]);
            out[(u64)d * n + e] = key;
            digits0[(u64)d * n + e] = (u8)key;
        }
        out[(u64)(words - 1) * n + e] = (u32)e;
    }
}

// Whether the four-points-per-thread variant fits k and the rows' alignment,
// and the kernel's name as the profiler prints it.
inline bool first_digits_vec(const float* pts, int k) {
    return k >= 1 && k <= 4 && reinterpret_cast<uintptr_t>(pts) % 16 == 0;
}
inline const char* first_digits_name(const float* pts, int k) {
    static const char* const names[5] = {"k_first_digits", "k_first_digits4<1>", "k_first_digits4<2>",
                                         "k_first_digits4<3>", "k_first_digits4<4>"};
    return first_digits_vec(pts, k) ? names[k] : names[0];
}

// Launches whichever of the two fits k and the rows' alignment.
void launch_first_digits(const float* pts, i64 n, int k, int kr, u8* digits0, hipStream_t stream) {
    const bool vec = first_digits_vec(pts, k);
    const i64 work = vec ? (n + 3) / 4 : (n > 0 ? n : 1);
    const unsigned grid = (unsigned)((work + kBlock - 1) / kBlock < (1 << 30) ? (work + kBlock - 1) / kBlock : (1 << 30));
    if (!vec) k_first_digits<<<grid, kBlock, 0, stream>>>(pts, n, k, kr, digits0);
    else if (k == 1) k_first_digits4<1><<<grid, kBlock, 0, stream>>>(pts, n, kr, digits0);
    else if (k == 2) k_first_digits4<2><<<grid, kBlock, 0, stream>>>(pts, n, kr, digits0);
    else if (k == 3) k_first_digits4<3><<<grid, kBlock, 0, stream>>>(pts, n, kr, digits0);
    else k_first_digits4<4><<<grid, kBlock, 0, stream>>>(pts, n, kr, digits0);
}

// Digit counts of the tiles of one chunk, from the pass's digit bytes (one
// byte read per record instead of the record).
__global__ __launch_bounds__(kCountBlock) void k_sort_count(SortArgs a) {
    __shared__ u32 hist[kCountBlock / 64][kRadix];
    __shared__ u32 rows[kChunkTiles][kRadix];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    // Counts do not depend on which thread counts which record: each thread
    // takes kPartItems consecutive records of its tile (one 8-byte load).
    const int g = tid / kSortBlock;  // tile of the chunk
    const i64 t = (i64)blockIdx.x * kChunkTiles + g;
    const i64 first = t * kSortTile + (i64)(tid % kSortBlock) * kPartItems;
    static_assert(kPartItems == 8, "one 8-byte load of digits per thread");
    u64 packed = 0;
    if (first + kPartItems <= a.src.n) {
        packed = *reinterpret_cast<const u64*>(a.digits + first);
    } else {
        for (int j = 0; j < kPartItems; ++j)
            if (first + j < a.src.n) packed |= (u64)a.digits[first + j] << (8 * j);
    }
    for (int i = lane; i < kRadix; i += 64) hist[w][i] = 0;  // this wave's own row
    // Each thread merges runs of equal digits among its own records first,
    // which keeps the skewed bytes of clustered keys off one counter.
    u32 last = 0, run = 0;
#pragma unroll
    for (int j = 0; j < kPartItems; ++j) {
        if (first + j >= a.src.n) break;
        const u32 d = (u32)(packed >> (8 * j)) & (kRadix - 1);
        if (run && d != last) {
            atomicAdd(&hist[w][last], run);
            run = 0;
        }
        last = d;
        ++run;
    }
    if (run) atomicAdd(&hist[w][last], run);
    __syncthreads();
    write_chunk_counts(hist, rows, kRadix, blockIdx.x, a.chunks, a.tiles, a.tile_counts,
                       a.chunk_counts);
}

template <int kSrc, int kW>
__global__ __launch_bounds__(kSortBlock) void k_sort_scatter(SortArgs a) {
    __shared__ union {
        u32 count[kSortWaves][kRadix];  // ranking: per-wave digit counts, then prefixes
        uint4 quads[kW == 4 ? kSortTile : 1];  // staging of the sorted tile
        uint2 pairs[kW == 2 ? kSortTile : 1];
        u32 words[kSortTile];
    } sm;
    __shared__ u8 s_digit[kSortTile];
    __shared__ u32 s_local[kRadix];  // first tile-local slot of each digit
    __shared__ u32 s_base[kRadix];   // global slot of tile-local slot 0 of each digit
    __shared__ u64 s_wave[kSortWaves];
    __shared__ u32 s_valid;          // records of the tile

    const u32 t = xcd_tile(a.tiles);
    if (t >= a.tiles) return;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const i64 wbase = (i64)t * kSortTile + (i64)w * (64 * kPartItems) + lane;
    RecordTile<kSrc, kW> tr;
    tr.load(a.src, wbase);
    // Thread tid < 256 owns digit tid: its records before this tile (its
    // chunk's prefix, plus the first tile's count in the chunk's second
    // tile, read with no branch), and the digit's total. With 16-byte
    // records the loads go out while the records are in flight; with
    // narrower ones (more workgroups per CU) after the digits.
    static_assert(kChunkTiles == 2, "two tiles per chunk");
    const bool owner = tid < kRadix;
    u32 global_start = 0, digit_total = 0;
    auto load_prefix = [&]() {
        const u32 c = t / kChunkTiles;
        const u32 chunk_before = a.chunk_counts[(u64)tid * a.chunks + c];
        const u32 first_tile = a.tile_counts[(u64)c * kChunkTiles * kRadix + tid];
        digit_total = a.totals[tid];
        global_start = chunk_before + ((t & 1) ? first_tile : 0u);
    };
    if constexpr (kW == 4)
        if (owner) load_prefix();
    u32 digit[kPartItems], rank[kPartItems];
    bool valid[kPartItems];
#pragma unroll
    for (int j = 0; j < kPartItems; ++j) {
        const i64 e = wbase + (i64)j * 64;
        valid[j] = e < a.src.n;
        digit[j] = valid[j] ? (tr.word(a.src, j, e, a.dim) >> a.shift) & (kRadix - 1) : 0u;
    }
    if constexpr (kW != 4)
        if (owner) load_prefix();
    for (int i = lane; i < kRadix; i += 64) sm.count[w][i] = 0;
    wave_rank(digit, valid, kRadixBits, sm.count[w], rank);
    __syncthreads();
    // Per-wave prefixes and the tile total of each digit.
    u32 agg = 0;
    if (owner) {
#pragma unroll
        for (int v = 0; v < kSortWaves; ++v) {
            const u32 c = sm.count[v][tid];
            sm.count[v][tid] = agg;
            agg += c;
        }
    }
    // Both exclusive scans at once: digit totals (high word) and the tile's
    // digit counts (low word, at most kSortTile in all).
    const u64 starts = block_exclusive_scan64<kSortWaves>(((u64)digit_total << 32) | agg, s_wave);
    if (owner) {
        const u32 local_start = (u32)starts;
        global_start += (u32)(starts >> 32);
        s_local[tid] = local_start;
        s_base[tid] = global_start - local_start;  // modular; base + slot < n
        if (tid == kRadix - 1) s_valid = local_start + agg;
    }
#pragma unroll
    for (int j = 0; j < kPartItems; ++j)
        if (valid[j]) rank[j] += sm.count[w][digit[j]];
    __syncthreads();  // s_local written, count reads done
    const int valid_here = (int)s_valid;
    // rank[j] becomes the record's slot in the tile's sorted order.
#pragma unroll
    for (int j = 0; j < kPartItems; ++j) {
        if (!valid[j]) continue;
        rank[j] += s_local[digit[j]];
        s_digit[rank[j]] = (u8)digit[j];
    }
    if constexpr (kW == 4) {
#pragma unroll
        for (int j = 0; j < kPartItems; ++j)
            if (valid[j]) sm.quads[rank[j]] = tr.quad(j);
        __syncthreads();
        for (int i = tid; i < valid_here; i += kSortBlock) {
            const u32 dst = s_base[s_digit[i]] + (u32)i;
            if (dst >= (u64)a.src.n) continue;
            const uint4 q = sm.quads[i];
            *reinterpret_cast<uint4*>(a.out + (u64)dst * 4) = q;
            if (a.next_digits) {
                const u32 c = (q.x & (a.next_dim == 0 ? ~0u : 0u)) | (q.y & (a.next_dim == 1 ? ~0u : 0u)) |
                              (q.z & (a.next_dim == 2 ? ~0u : 0u));
                a.next_digits[dst] = (u8)(c >> a.next_shift);
            }
        }
    } else if constexpr (kW == 2) {
#pragma unroll
        for (int j = 0; j < kPartItems; ++j)
            if (valid[j]) sm.pairs[rank[j]] = make_uint2(tr.template at<0>(j), tr.template at<1>(j));
        __syncthreads();
        for (int i = tid; i < valid_here; i += kSortBlock) {
            const u32 dst = s_base[s_digit[i]] + (u32)i;
            if (dst >= (u64)a.src.n) continue;
            const uint2 v = sm.pairs[i];
            *reinterpret_cast<uint2*>(a.out + (u64)dst * 2) = v;
            if (a.next_digits) a.next_digits[dst] = (u8)((a.next_dim == 0 ? v.x : v.y) >> a.next_shift);
        }
    } else {
        // one word of every record per staging round; wide records (kW = 0)
        // are read from the source a round ahead, so that the loads of word
        // ww + 1 are in flight during round ww
        const int words = kW > 0 ? kW : a.src.words;
        u32 next[kPartItems];
#pragma unroll
        for (int j = 0; j < kPartItems; ++j) next[j] = valid[j] ? tr.word(a.src, j, wbase + (i64)j * 64, 0) : 0u;
        for (int ww = 0; ww < words; ++ww) {
            __syncthreads();  // the previous round's reads are done
#pragma unroll
            for (int j = 0; j < kPartItems; ++j)
                if (valid[j]) sm.words[rank[j]] = next[j];
            if (ww + 1 < words) {
#pragma unroll
                for (int j = 0; j < kPartItems; ++j)
                    next[j] = valid[j] ? tr.word(a.src, j, wbase + (i64)j * 64, ww + 1) : 0u;
            }
            __syncthreads();
            for (int i = tid; i < valid_here; i += kSortBlock) {
                const u32 dst = s_base[s_digit[i]] + (u32)i;
                if (dst >= (u64)a.src.n) continue;
                a.out[rec_word_index(words, a.src.plane, dst, ww)] = sm.words[i];
                if (ww == a.next_dim && a.next_digits)
                    a.next_digits[dst] = (u8)(sm.words[i] >> a.next_shift);
            }
        }
    }
}

// ------------------------------------- re-sort by tag: the per-round pass
// Array `in` holds the records of the points still live on level l0 (not
// yet a node above it) in round-l0 order: segment j of level l0 at live
// positions [live_begin(j), live_begin(j+1)), each sorted by (coordinate,
// index). The pass moves every point to its segment on level l1 = l0 +
// delta, keeping the order inside each segment; the pivots of the levels in
// between drop out (they are nodes already). A point's digit is the offset
// of its level-l1 node below its level-l0 node (delta bits); its output
// position is
//   live_begin(its level-l1 node)
//   + (points of its digit before it in `in`)
//   - (those in earlier level-l0 segments: bin_prefix, closed form).
struct PartArgs {
    RecordSource src;  // records live on level l0 (src.n of them)
    u32* out;          // records live on level l1: n_out x words
    i64 n_out;
    int k;             // dimensions: level l splits coordinate l mod k
    int l0, l1;        // levels before and after (1 <= l1 - l0 <= kMaxDescent)
    int dim0;          // l0 mod k
    Geometry geo;
    LevelShape s0, s1; // the closed-form constants of levels l0 and l1
    const u64* piv;    // pivot of node s: key(coordinate) << 32 | index
    u32 tiles;
    u32* chunk_counts; // bins x tiles: digit counts of each tile, then the
                       //   counts of the digit in the tiles before it
    // When l1 is the round's level, the pass also fixes that level's nodes:
    // the record whose rank in its new segment is the left subtree's size
    // is the node's pivot ([W], sb/ss paragraph).
    u64* piv_out;      // pivot table, or nullptr for an intermediate pass
    int dim1;          // l1 mod k
    LevelShape s2;     // closed-form constants of level l1 + 1
    int32_t* perm;     // optional outputs for the nodes of level l1
    float* tree;
    // Split-widest-dimension trees: every node's split dimension (nullptr:
    // level mod k). The array is sorted by coordinate array_dim, so the pass
    // fixes only the level-l1 nodes that split it; leaf_level: l1 is the
    // last level, whose nodes have empty subtrees below them.
    const uint16_t* dimtab;
    int array_dim;
    int leaf_level;
    // Select passes of split-widest trees: bit d of level_dims[l1] says some
    // level-l1 node splits dimension d (nullptr: do not skip); without one
    // for array_dim the pass has no pivot to find and its kernels return.
    const u32* level_dims;
};

// Whether a select pass of a split-widest tree has nothing to do.
__device__ __forceinline__ bool no_nodes_here(const PartArgs& a) {
    return a.level_dims && !((a.level_dims[a.l1] >> a.array_dim) & 1u);
}

// Pivots one tile's walk keeps in LDS: the nodes of levels l0 .. l1-1 below
// the level-l0 segments the tile overlaps (2 of them at most while segments
// are as long as a tile, 2^delta - 1 nodes below each). Round-robin trees
// only: split-widest walks read the pivots and node dimensions in place
// (staging measured slower there).
constexpr int kPivStage = 1024;

// One level of the walk for round-robin trees, whose level dimension kD is
// the same for the whole wave: the compared words are picked at compile
// time. piv_level[loc] is the pivot of the item's node; only valid items
// read it.
template <int kD, int kW, typename Piv>
__device__ __forceinline__ void walk_level(const RecordTile<kSrcRecords, kW>& tr, Piv piv_level,
                                           u32 (&loc)[kPartItems], bool (&valid)[kPartItems]) {
#pragma unroll
    for (int j = 0; j < kPartItems; ++j) {
        const u64 me = ((u64)tr.template at<kD>(j) << 32) | tr.template at<kW - 1>(j);
        const u64 p = valid[j] ? piv_level[loc[j]] : 0;
        if (me == p) valid[j] = false;  // the pivot itself: a node already
        loc[j] = 2 * loc[j] + (me < p ? 0u : 1u);
    }
}

// One step of a walk kept as r = ~loc: the next node is 2 loc + (me >= p),
// so ~loc' = 2 r + (me < p), and (me < p) is the borrow of the 64-bit
// subtraction (key:index) - (pivot key:pivot index). Three 32-bit ALU
// instructions on the words as they are; compiled code would pair the words
// into 64-bit registers and materialise the comparison bit instead.
__device__ __forceinline__ u32 walk_step(u32 r, u32 key, u32 index, u32 pkey, u32 pindex) {
    u32 diff;
    u64 borrow;
    asm("v_sub_co_u32_e64 %1, %2, %3, %5\n\t"
        "v_subb_co_u32_e64 %1, %2, %4, %6, %2\n\t"
        "v_addc_co_u32_e64 %0, %2, %0, %0, %2"
        : "+v"(r), "=&v"(diff), "=&s"(borrow)
        : "v"(index), "v"(key), "v"(pindex), "v"(pkey));
    return r;
}

// One level of a walk over staged pivots, stored in reverse within the
// level: the pivot of loc sits at level_end[-1 - loc] = level_end[r]. Every
// item's r is in range (past-the-end items walk from slot 0), so the read
// needs no mask. The pivot itself is found by its index word alone (indices
// are unique, and its key is the compared one).
template <int kD, int kW>
__device__ __forceinline__ void walk_level_staged(const RecordTile<kSrcRecords, kW>& tr, const u64* level_end,
                                                  u32 (&r)[kPartItems], bool (&valid)[kPartItems]) {
#pragma unroll
    for (int j = 0; j < kPartItems; ++j) {
        const u64 p = level_end[(int)r[j]];
        const u32 index = tr.template at<kW - 1>(j);
        if (index == (u32)p) valid[j] = false;  // the pivot itself: a node already
        r[j] = walk_step(r[j], tr.template at<kD>(j), index, (u32)(p >> 32), (u32)p);
    }
}

// a where the lane's bit of `mask` is clear, else b: one v_cndmask. Written
// out because a chain of such selects among a thread's record words is
// otherwise compiled into an indexed load from a scratch copy of them.
__device__ __forceinline__ u32 pick_lanes(u32 a, u32 b, u64 mask) {
    u32 r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(mask));
    return r;
}

// The same for split-widest trees: each node's split dimension is staged
// beside its pivot (reversed the same way) and picks the compared key.
template <int kW>
__device__ __forceinline__ void walk_level_staged_dims(const RecordTile<kSrcRecords, kW>& tr, const u64* level_end,
                                                       const uint8_t* dims_end, u32 (&r)[kPartItems],
                                                       bool (&valid)[kPartItems]) {
#pragma unroll
    for (int j = 0; j < kPartItems; ++j) {
        const u64 p = level_end[(int)r[j]];
        const u32 dj = dims_end[(int)r[j]];
        const u32 index = tr.template at<kW - 1>(j);
        // (lane masks of dj == 1 and dj == 2; ICMP_EQ = 32)
        u32 key = tr.template at<0>(j);
        if constexpr (kW > 2) key = pick_lanes(key, tr.template at<1>(j), __builtin_amdgcn_uicmp(dj, 1u, 32));
        if constexpr (kW > 3) key = pick_lanes(key, tr.template at<2>(j), __builtin_amdgcn_uicmp(dj, 2u, 32));
        if (index == (u32)p) valid[j] = false;  // the pivot itself: a node already
        r[j] = walk_step(r[j], key, index, (u32)(p >> 32), (u32)p);
    }
}

template <int kW, int kM>
__device__ __forceinline__ void walk_staged_dims(const RecordTile<kSrcRecords, kW>& tr, const u64* s_piv,
                                                 const uint8_t* s_dim, u32 segs, int delta, u32 (&r)[kPartItems],
                                                 bool (&valid)[kPartItems]) {
    if constexpr (kM < kMaxDescent) {
        if (kM >= delta) return;
        const u32 end = segs * ((2u << kM) - 1);
        walk_level_staged_dims<kW>(tr, s_piv + end, s_dim + end, r, valid);
        walk_staged_dims<kW, kM + 1>(tr, s_piv, s_dim, segs, delta, r, valid);
    }
}

// Levels kM .. delta-1 of a walk over staged pivots, the dimension of level
// l0 + m being (kD0 + m) mod (kW - 1) at compile time (records of kW words
// hold kW - 1 keys, one per dimension). Level m's pivots end at slot
// segs * (2^(m+1) - 1).
template <int kD0, int kW, int kM>
__device__ __forceinline__ void walk_staged(const RecordTile<kSrcRecords, kW>& tr, const u64* s_piv, u32 segs,
                                            int delta, u32 (&r)[kPartItems], bool (&valid)[kPartItems]) {
    if constexpr (kM < kMaxDescent) {
        if (kM >= delta) return;
        walk_level_staged<(kD0 + kM) % (kW - 1), kW>(tr, s_piv + segs * ((2u << kM) - 1), r, valid);
        walk_staged<kD0, kW, kM + 1>(tr, s_piv, segs, delta, r, valid);
    }
}

// The walk one level at a time, for records without registers (kW = 0) and
// for pivots read in place: compare with the pivot of the current node, in
// the level's dimension (or the node's own, from the table).
template <int kW, bool kNodeDims, bool kInPlace, int kIdx>
__device__ __forceinline__ void part_nodes_loop(const PartArgs& a, const RecordTile<kSrcRecords, kW>& tr, i64 wbase,
                                                u32 j_first, u32 segs, bool staged, const u64* s_piv,
                                                const u32 (&index_of)[kIdx], u32 (&loc)[kPartItems],
                                                bool (&valid)[kPartItems]) {
    const int delta = a.l1 - a.l0;
    int dim = a.dim0;
    for (int m = 0; m < delta; ++m) {
        const u32 slot0 = segs * ((1u << m) - 1);
        const u32 node0 = (u32)(full_nodes(a.l0 + m) + ((u64)j_first << m));  // n < 2^31
        (void)slot0;
        if constexpr (kW > 0 && !kNodeDims && kInPlace) {
            constexpr int kD1 = kW > 2 ? 1 : 0, kD2 = kW > 3 ? 2 : 0;
            const u64* lv = a.piv + node0;  // (unstaged: read in place)
            if (dim == 0) walk_level<0, kW>(tr, lv, loc, valid);
            else if (dim == 1) walk_level<kD1, kW>(tr, lv, loc, valid);
            else walk_level<kD2, kW>(tr, lv, loc, valid);
        } else {
#pragma unroll
            for (int j = 0; j < kPartItems; ++j) {
                const i64 e = wbase + (i64)j * 64;
                int dj = dim;
                u64 p = 0;
                if (valid[j]) {
                    p = staged ? s_piv[slot0 + loc[j]] : a.piv[node0 + loc[j]];
                    if constexpr (kNodeDims) dj = (int)a.dimtab[node0 + loc[j]];
                } else if constexpr (kNodeDims) {
                    dj = 0;
                }
                const u64 me = ((u64)tr.word(a.src, j, e, dj) << 32) | index_of[j];
                if (me == p) valid[j] = false;  // the pivot itself: a node already
                loc[j] = 2 * loc[j] + (me < p ? 0u : 1u);
            }
        }
        if (++dim == a.k) dim = 0;
    }
}

// For every item: node[j], the in-level index of its node on level l1,
// which is (j0 << delta) | digit for its level-l0 segment j0 and its digit
// (offset of the level-l1 node below the level-l0 one); valid = false for
// records past the end and for the pivots of levels l0 .. l1-1. The walk
// compares (key(coordinate l mod k), index) with the pivot of the current
// node on each level l ([W], tag paragraph: before the pivot -> left child).
// Call with the whole workgroup: the pivots are staged in LDS first.
// Records held in registers (kW > 0) always stage them, with the node
// dimensions of split-widest trees (the host checks that every tile's fit:
// pivots_fit), unless kInPlace: then the walk reads them where they are.
template <int kW, bool kNodeDims, bool kInPlace = false>
__device__ __forceinline__ void part_nodes(const PartArgs& a, u32 t,
                                           const RecordTile<kSrcRecords, kW>& tr, i64 wbase,
                                           u32 (&node)[kPartItems], bool (&valid)[kPartItems]) {
    // (records held in registers walk each level's pivots in reverse)
    constexpr bool kReversed = kW > 0 && !kInPlace;
    __shared__ u64 s_piv[kInPlace || (kNodeDims && !kReversed) ? 1 : kPivStage];
    __shared__ uint8_t s_dim[kNodeDims && kReversed ? kPivStage : 1];
    const int delta = a.l1 - a.l0;
    const u64 p0 = (u64)t * kPartTile;
    const u64 p1 = p0 + kPartTile < (u64)a.src.n ? p0 + kPartTile : (u64)a.src.n;
    const u32 j_first = (u32)live_segment(a.geo, p0, a.l0);
    const u32 segs = (u32)live_segment(a.geo, p1 - 1, a.l0) - j_first + 1;
    // Level l0 + m of the walk: nodes (j_first << m) + i, i < segs << m, at
    // slots segs * (2^m - 1) + i (nodes past the last leaf: never visited).
    const u32 staged_n = segs * ((1u << delta) - 1);
    const bool staged = kReversed || (!kNodeDims && !kInPlace && staged_n <= (u32)kPivStage);
    if (staged) {
        const u32 stage_n = staged_n < (u32)kPivStage ? staged_n : (u32)kPivStage;
        for (u32 s = threadIdx.x; s < stage_n; s += kBlock) {
            const int m = 31 - __clz(s / segs + 1);
            const u32 i = s - segs * ((1u << m) - 1);
            const u64 nd = full_nodes(a.l0 + m) + ((u64)j_first << m) + i;
            const bool real = nd < (u64)a.geo.n;
            const u32 slot = kReversed ? segs * ((2u << m) - 1) - 1 - i : s;
            s_piv[slot] = real ? a.piv[nd] : 0;
            if constexpr (kNodeDims && kReversed) s_dim[slot] = real ? (uint8_t)a.dimtab[nd] : (uint8_t)0;
        }
    }
    // Level-l0 segment of each record: one division for the wave's first
    // record, then each lane steps over the segment starts it passes (its
    // records are 64 positions apart, in increasing order). loc: the node's
    // in-level index less j_first << m.
    const u32 wfirst = (u32)(wbase - (threadIdx.x & 63));
    u32 j0 = (u32)live_segment(a.geo, wfirst, a.l0);
    u32 next = live_begin32(a.s0, j0 + 1);
    u32 loc[kPartItems];
#pragma unroll
    for (int j = 0; j < kPartItems; ++j) {
        const u32 e = (u32)(wbase + (i64)j * 64);
        valid[j] = e < (u64)a.src.n;
        if (valid[j]) {
            while (e >= next) {
                ++j0;
                next = live_begin32(a.s0, j0 + 1);
            }
        }
        // past the end: slot 0, so that every loc stays below segs << m
        loc[j] = valid[j] ? j0 - j_first : 0u;
    }
    // (records without registers: the index word once per item)
    u32 index_of[kReversed || (kW > 0 && !kNodeDims) ? 1 : kPartItems];
    if constexpr (!(kReversed || (kW > 0 && !kNodeDims))) {
#pragma unroll
        for (int j = 0; j < kPartItems; ++j) {
            const i64 e = wbase + (i64)j * 64;
            index_of[j] = valid[j] ? tr.word(a.src, j, e, a.src.words - 1) : 0u;
        }
    }
    if (staged) __syncthreads();
    if constexpr (kReversed) {  // levels unrolled
#pragma unroll
        for (int j = 0; j < kPartItems; ++j) loc[j] = ~loc[j];
        if constexpr (kNodeDims) {
            walk_staged_dims<kW, 0>(tr, s_piv, s_dim, segs, delta, loc, valid);
        } else {  // dimensions fixed at compile time
            constexpr int kK = kW - 1;
            if (a.dim0 == 0) walk_staged<0, kW, 0>(tr, s_piv, segs, delta, loc, valid);
            else if (a.dim0 == 1) walk_staged<1 % kK, kW, 0>(tr, s_piv, segs, delta, loc, valid);
            else walk_staged<2 % kK, kW, 0>(tr, s_piv, segs, delta, loc, valid);
        }
#pragma unroll
        for (int j = 0; j < kPartItems; ++j) node[j] = (j_first << delta) + ~loc[j];
    } else {
        part_nodes_loop<kW, kNodeDims, kInPlace>(a, tr, wbase, j_first, segs, staged, s_piv, index_of, loc, valid);
#pragma unroll
        for (int j = 0; j < kPartItems; ++j) node[j] = (j_first << delta) + loc[j];
    }
}

// Digit counts of one tile of a re-sort pass. A re-sort pass has at most
// 2^kMaxDescent digits, usually a handful, so every tile is its own chunk:
// its count of digit d goes straight to row d of the digit-major counts.
template <int kW, bool kNodeDims, bool kInPlace = false>
__device__ __forceinline__ void part_count_tile(const PartArgs& a, u32 t) {
    __shared__ u32 hist[kWaves][kRadix];
    if (t >= a.tiles) return;
    if constexpr (kNodeDims)
        if (no_nodes_here(a)) return;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const i64 wbase = (i64)t * kPartTile + (i64)w * (64 * kPartItems) + lane;
    const int bins = 1 << (a.l1 - a.l0);
    RecordTile<kSrcRecords, kW> tr;
    if constexpr (kW > 0) tr.load_all(a.src, wbase);
    else tr.load(a.src, wbase);
    u32 node[kPartItems];
    bool valid[kPartItems];
    part_nodes<kW, kNodeDims, kInPlace>(a, t, tr, wbase, node, valid);
    for (int i = lane; i < bins; i += 64) hist[w][i] = 0;  // this wave's own row
    u32 last = 0, run = 0;
#pragma unroll
    for (int j = 0; j < kPartItems; ++j) {
        if (!valid[j]) continue;
        const u32 digit = node[j] & (bins - 1);
        if (run && digit != last) {
            atomicAdd(&hist[w][last], run);
            run = 0;
        }
        last = digit;
        ++run;
    }
    if (run) atomicAdd(&hist[w][last], run);
    __syncthreads();
    if (tid < bins) {
        u32 total = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) total += hist[v][tid];
        a.chunk_counts[(u64)tid * a.tiles + t] = total;
    }
}

template <int kW, bool kNodeDims, bool kInPlace = false>
__device__ __forceinline__ void part_count(const PartArgs& a) {
    part_count_tile<kW, kNodeDims, kInPlace>(a, xcd_tile(a.tiles));
}

// Split dimension l mod k (round-robin trees) / from the node table
// (split-widest trees).
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_count(PartArgs a) { part_count<kW, false>(a); }
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_count_widest(PartArgs a) { part_count<kW, true>(a); }
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_count_inplace(PartArgs a) { part_count<kW, false, true>(a); }
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_count_widest_inplace(PartArgs a) { part_count<kW, true, true>(a); }

// Whether tile t of a pass holds the pivot of some level-l1 node. The node
// with in-level index j0 * 2^delta + b has its pivot where the count of
// digit-b records before it reaches bin_prefix(j0, b) + |S(left child)|, and
// tile t holds the digit-b records counted from chunk_counts[b][t] up to
// chunk_counts[b][t+1] (the last tile: all the rest). Only the level-l0
// segments the tile overlaps can have their pivots in it.
template <bool kNodeDims>
__device__ bool tile_has_pivot(const PartArgs& a, u32 t) {
    const int delta = a.l1 - a.l0;
    const u32 bins = 1u << delta;
    const u64 p0 = (u64)t * kPartTile;
    const u64 p1 = p0 + kPartTile < (u64)a.src.n ? p0 + kPartTile : (u64)a.src.n;
    const u32 j_first = (u32)live_segment(a.geo, p0, a.l0);
    const u32 j_last = (u32)live_segment(a.geo, p1 - 1, a.l0);
    const u32 pairs = (j_last - j_first + 1) << delta;
    const bool tail = t + 1 == a.tiles;
    int hit = 0;
    for (u32 i = threadIdx.x; i < pairs; i += kBlock) {
        const u32 j0 = j_first + (i >> delta), b = i & (bins - 1);
        const u32 node = (j0 << delta) | b;
        if (full_nodes(a.l1) + node >= (u64)a.geo.n) continue;  // past the last leaf
        if constexpr (kNodeDims)  // another array's node
            if (a.dimtab[full_nodes(a.l1) + node] != (uint16_t)a.array_dim) continue;
        const u32 left = a.leaf_level ? 0u : subtree_size32(a.s2, 2 * node);
        const u32 target = bin_prefix32(a.s1, j0, b, delta) + left;
        const u32* row = a.chunk_counts + (u64)b * a.tiles;
        if (target >= row[t] && (tail || target < row[t + 1])) hit = 1;
    }
    return __syncthreads_or(hit) != 0;
}

// The tile of a pass that holds the pivot of level-l1 node i = j0 * 2^delta
// + b: the pivot is the record where the count of digit-b records reaches
// bin_prefix(j0, b) + |S(left child)|, and tile t holds the digit-b records
// counted from chunk_counts[b][t] (scanned: the count before the tile) up to
// chunk_counts[b][t+1], so the pivot's tile is the last t whose count before
// it is at most that target. Only the tiles of segment j0 can hold it; they
// are searched 256 probes at a time, one every `stride` tiles, each round
// narrowing the range to the stride the target fell in, until one tile is
// left. Call with the whole workgroup.
__device__ u32 pivot_tile(const PartArgs& a, u32 i) {
    const int delta = a.l1 - a.l0;
    const u32 j0 = i >> delta, b = i & ((1u << delta) - 1);
    const u32 left = a.leaf_level ? 0u : subtree_size32(a.s2, 2 * i);
    const u32 target = bin_prefix32(a.s1, j0, b, delta) + left;
    const u32* row = a.chunk_counts + (u64)b * a.tiles;
    const u32 t_lo = live_begin32(a.s0, j0) / kPartTile;
    const u32 end = live_begin32(a.s0, j0 + 1);  // (a segment is never empty)
    u32 t_hi = (end - 1) / kPartTile;
    if (t_hi >= a.tiles) t_hi = a.tiles - 1;
    // Counts before the tiles do not decrease, and the first tile's is at
    // most the target (only earlier segments' records precede it): of the
    // probes, those at most the target are a leading run of at least one.
    u32 lo = t_lo, len = t_hi - t_lo + 1;
    while (len > 1) {
        const u32 stride = (len + kBlock - 1) / kBlock;
        const u32 probe = lo + threadIdx.x * stride;
        const u32 c = (u32)__syncthreads_count(probe < lo + len && row[probe] <= target);
        lo += (c - 1) * stride;
        const u32 rest = t_hi + 1 - lo;
        len = stride < rest ? stride : rest;
    }
    return lo;
}

// kSelect: the pass only fixes the level-l1 nodes; it reads the tiles that
// hold their pivots and writes no records (the array keeps its level-l0
// order, and its next re-sort walks the levels in between as well).
// only: for a select, the in-level index of the one node whose pivot this
// workgroup writes, or kEveryNode: every pivot in the tile (of this array's
// dimension, for split-widest trees).
constexpr u32 kEveryNode = ~0u;
template <int kW, bool kNodeDims, bool kSelect, bool kInPlace>
__device__ __forceinline__ void part_tile(const PartArgs& a, u32 t, u32 only) {
    __shared__ u32 count[kWaves][kRadix];  // per-wave digit counts, then first slots
    // Wide (planar) records of a re-sort are staged in LDS in output order
    // and written a word plane at a time as the tile's runs: written record
    // by record, each store of a wave would touch up to 64 lines per plane.
    constexpr bool kStage = kW == 0 && !kSelect;
    __shared__ u32 s_words[kStage ? kPartTile : 1];  // one word of each staged record
    __shared__ u32 s_pos[kStage ? kPartTile : 1];    // its output position (~0: none)
    __shared__ u32 s_first[kStage ? kRadix : 1];     // tile slot of a digit's first record, less
                                                     //   the digit's count before the tile
    __shared__ u32 s_scan[kWaves];
    __shared__ u32 s_staged;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const i64 wbase = (i64)t * kPartTile + (i64)w * (64 * kPartItems) + lane;
    const int delta = a.l1 - a.l0;
    const int bins = 1 << delta;
    RecordTile<kSrcRecords, kW> tr;
    if constexpr (kW > 0) tr.load_all(a.src, wbase);
    else tr.load(a.src, wbase);
    // points of digit tid before the tile (loaded while the records are in flight)
    const u32 before_tile = tid < bins ? a.chunk_counts[(u64)tid * a.tiles + t] : 0u;
    u32 node[kPartItems], rank[kPartItems];
    bool valid[kPartItems];
    part_nodes<kW, kNodeDims, kInPlace>(a, t, tr, wbase, node, valid);
    for (int i = lane; i < bins; i += 64) count[w][i] = 0;
    {
        u32 digit[kPartItems];
#pragma unroll
        for (int j = 0; j < kPartItems; ++j) digit[j] = node[j] & (bins - 1);
        wave_rank(digit, valid, delta, count[w], rank);
    }
    __syncthreads();
    u32 tile_total = 0;
    if (tid < bins) {
        // points of this digit before the tile, then before each wave
        u32 run = before_tile;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const u32 c = count[v][tid];
            count[v][tid] = run;
            run += c;
        }
        tile_total = run - before_tile;
    }
    if constexpr (kStage) {
        // (the scan's own barriers also order the counts above)
        const u32 start = block_exclusive_scan(tile_total, s_scan);
        if (tid < bins) s_first[tid] = start - before_tile;
        if (tid == bins - 1) s_staged = start + tile_total;
    }
    __syncthreads();
    u32 slot[kStage ? kPartItems : 1];
#pragma unroll
    for (int j = 0; j < kPartItems; ++j) {
        if (!valid[j]) continue;
        const u32 digit = node[j] & (bins - 1);
        const u32 in_segment = count[w][digit] + rank[j] - bin_prefix32(a.s1, node[j] >> delta, digit, delta);
        const i64 e = wbase + (i64)j * 64;
        if constexpr (kStage) {
            const u32 pos = live_begin32(a.s1, node[j]) + in_segment;
            slot[j] = s_first[digit] + count[w][digit] + rank[j];
            s_pos[slot[j]] = pos < (u64)a.n_out ? pos : ~0u;
        } else if constexpr (!kSelect) {
            const u32 pos = live_begin32(a.s1, node[j]) + in_segment;
            if (pos < (u64)a.n_out) {
                // non-temporal while a wave's records fall in few runs, plain
                // once the walk spreads them over 2^kPlainDelta or more
                if (delta >= kPlainDelta) tr.store_plain(a.src, a.out, j, e, pos);
                else tr.store(a.src, a.out, j, e, pos);
            }
        }
        const u32 left = a.leaf_level ? 0u : subtree_size32(a.s2, 2 * node[j]);
        bool mine = true;  // the node splits this array's dimension
        if (kSelect && only != kEveryNode) mine = node[j] == only;  // (whose dimension the caller checked)
        else if constexpr (kNodeDims) mine = a.dimtab[full_nodes(a.l1) + node[j]] == (uint16_t)a.array_dim;
        if (a.piv_out && in_segment == left && mine) {
            const u64 s = full_nodes(a.l1) + node[j];
            const u32 idx = tr.word(a.src, j, e, a.src.words - 1);
            a.piv_out[s] = ((u64)tr.word(a.src, j, e, a.dim1) << 32) | idx;
            if (a.perm) a.perm[s] = (int32_t)idx;
            // (the row from `points`: a key does not keep the sign of zero)
            if (a.tree)
                for (int d = 0; d < a.k; ++d) a.tree[s * a.k + d] = a.src.pts[(u64)idx * a.k + d];
        }
    }
    if constexpr (kStage) {
        const u32 staged = s_staged;  // (written before the barrier above)
        // each word read a round ahead (its loads in flight meanwhile)
        u32 next[kPartItems];
#pragma unroll
        for (int j = 0; j < kPartItems; ++j) next[j] = valid[j] ? tr.word(a.src, j, wbase + (i64)j * 64, 0) : 0u;
        for (int ww = 0; ww < a.src.words; ++ww) {
            __syncthreads();  // positions written; the previous round's reads done
#pragma unroll
            for (int j = 0; j < kPartItems; ++j)
                if (valid[j]) s_words[slot[j]] = next[j];
            if (ww + 1 < a.src.words) {
#pragma unroll
                for (int j = 0; j < kPartItems; ++j)
                    next[j] = valid[j] ? tr.word(a.src, j, wbase + (i64)j * 64, ww + 1) : 0u;
            }
            __syncthreads();
            for (u32 i = tid; i < staged; i += kBlock) {
                const u32 pos = s_pos[i];
                if (pos != ~0u) a.out[rec_word_index(a.src.words, a.src.plane, pos, ww)] = s_words[i];
            }
        }
    }
}

template <int kW, bool kNodeDims, bool kInPlace = false>
__device__ __forceinline__ void part_scatter(const PartArgs& a) {
    const u32 t = xcd_tile(a.tiles);
    if (t >= a.tiles) return;
    part_tile<kW, kNodeDims, false, kInPlace>(a, t, 0);
}

// A select: one workgroup per node of level l1 (of this array's dimension,
// for split-widest trees), on the tile that holds its pivot.
template <int kW, bool kNodeDims, bool kInPlace = false>
__device__ __forceinline__ void part_select(const PartArgs& a) {
    const u32 i = blockIdx.x;
    if (full_nodes(a.l1) + i >= (u64)a.geo.n) return;
    if constexpr (kNodeDims)
        if (a.dimtab[full_nodes(a.l1) + i] != (uint16_t)a.array_dim) return;
    part_tile<kW, kNodeDims, true, kInPlace>(a, pivot_tile(a, i), i);
}

// A select over levels with more nodes: one workgroup per tile, those that
// hold pivots writing them all.
template <int kW, bool kNodeDims, bool kInPlace = false>
__device__ __forceinline__ void part_select_tiles(const PartArgs& a) {
    const u32 t = xcd_tile(a.tiles);
    if (t >= a.tiles) return;
    if constexpr (kNodeDims)
        if (no_nodes_here(a)) return;
    if (!tile_has_pivot<kNodeDims>(a, t)) return;
    part_tile<kW, kNodeDims, true, kInPlace>(a, t, kEveryNode);
}

template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_scatter(PartArgs a) { part_scatter<kW, false>(a); }
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_scatter_widest(PartArgs a) { part_scatter<kW, true>(a); }
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_select(PartArgs a) { part_select<kW, false>(a); }
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_select_widest(PartArgs a) { part_select<kW, true>(a); }
// Round-robin passes whose tiles' pivots may not fit the LDS stage.
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_scatter_inplace(PartArgs a) { part_scatter<kW, false, true>(a); }
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_select_inplace(PartArgs a) { part_select<kW, false, true>(a); }
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_scatter_widest_inplace(PartArgs a) { part_scatter<kW, true, true>(a); }
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_select_widest_inplace(PartArgs a) { part_select<kW, true, true>(a); }
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_select_tiles(PartArgs a) { part_select_tiles<kW, false>(a); }
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_select_tiles_inplace(PartArgs a) { part_select_tiles<kW, false, true>(a); }
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_select_tiles_widest(PartArgs a) { part_select_tiles<kW, true>(a); }
template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_select_tiles_widest_inplace(PartArgs a) {
    part_select_tiles<kW, true, true>(a);
}

// Up to kMaxBatch passes of one split-widest level (one per array) in one
// launch per kernel: pass i owns blocks [first[i], first[i+1]) of the grid.
// Count and select kernels are short next to their launch and drain, so a
// level's passes share them.
constexpr int kMaxBatch = 4;
struct PartBatch {
    PartArgs a[kMaxBatch];
    u32 first[kMaxBatch + 1];  // first block of each pass (count: multiples of kXcds)
    u32 rows[kMaxBatch + 1];   // first scan row of each pass (its digits)
    int count;
};
static_assert(sizeof(PartBatch) <= 4096, "a kernel argument");

__device__ __forceinline__ int batch_pass(const u32 (&first)[kMaxBatch + 1], int count, u32& local) {
    int i = 0;
    while (i + 1 < count && blockIdx.x >= first[i + 1]) ++i;
    local = blockIdx.x - first[i];
    return i;
}

template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_count_widest_batch(PartBatch b) {
    u32 local;
    const int i = batch_pass(b.first, b.count, local);
    part_count_tile<kW, true>(b.a[i], xcd_tile_of(local, b.a[i].tiles));
}

template <int kW>
__global__ __launch_bounds__(kBlock) void k_part_select_widest_batch(PartBatch b) {
    u32 local;
    const int i = batch_pass(b.first, b.count, local);
    const PartArgs& a = b.a[i];
    if (full_nodes(a.l1) + local >= (u64)a.geo.n) return;
    if (a.dimtab[full_nodes(a.l1) + local] != (uint16_t)a.array_dim) return;
    part_tile<kW, true, true, false>(a, pivot_tile(a, local), local);
}

// Each pass's digit rows of tile counts, one workgroup a row (of kThreads:
// 1024 where a row is longer than one stretch of 256 threads).
template <int kThreads>
__global__ __launch_bounds__(kThreads) void k_chunk_scan_batch(PartBatch b) {
    u32 row;
    const int i = batch_pass(b.rows, b.count, row);
    const PartArgs& a = b.a[i];
    chunk_scan_row<kThreads>(a.chunk_counts + (u64)row * a.tiles, (i64)a.tiles, nullptr, 0);
}

// Round l's nodes: the pivot of node s = F(l) + j is the record at live
// position live_begin(j) + |S(2s+1)| of the array sorted for round l
// ([W], sb/ss paragraph). It goes to the pivot table, perm and tree.
__global__ __launch_bounds__(kBlock) void k_pivots(const u32* __restrict__ recs, int words, u64 plane,
                                                   Geometry geo, int l, int dim,
                                                   u64* __restrict__ piv,
                                                   const float* __restrict__ pts, int k,
                                                   int32_t* __restrict__ perm,
                                                   float* __restrict__ tree,
                                                   const uint16_t* __restrict__ dimtab) {
    const u64 j = (u64)blockIdx.x * kBlock + threadIdx.x;
    if (j >= (1ull << l)) return;
    const u64 s = full_nodes(l) + j;
    const u64 p = live_begin(geo, j, l) + subtree_size(geo, 2 * s + 1);
    if (s >= (u64)geo.n || p >= (u64)geo.n - full_nodes(l)) return;  // not for l < L-1
    if (dimtab && dimtab[s] != (uint16_t)dim) return;  // another array's node
    const u32 idx = recs[rec_word_index(words, plane, p, words - 1)];
    piv[s] = ((u64)recs[rec_word_index(words, plane, p, dim)] << 32) | idx;
    if (perm) perm[s] = (int32_t)idx;
    if (tree && idx < (u64)geo.n)
        for (int d = 0; d < k; ++d) tree[s * k + d] = pts[(u64)idx * k + d];
}

// Rounds by per-point tags (tag_rounds: many dimensions, whose arrays would
// each cost a pass a round): each point keeps the node it is in as a 32-bit
// tag, in index order, with kFixedTag set once it is its node's pivot. Round
// l brings every tag from level l-1 to level l (the point against its node's
// pivot by (key, index) in dimension (l-1) mod k: the left child below it,
// the right one above), then writes the point's record for the round's sort:
// (key in dimension l mod k, node offset on level l, 0, index),
// a fixed point's node offset ~0 so that it sorts after every live one
// ([W], tag paragraph: the tag is the node; sort order paragraph).
constexpr u32 kFixedTag = 0x80000000u;

__device__ __forceinline__ u32 tag_descend(u32 t, u32 key, u32 p, const u64* __restrict__ piv) {
    if (t & kFixedTag) return t;
    const u64 me = ((u64)key << 32) | p, pv = piv[t];
    return me == pv ? (t | kFixedTag) : (me < pv ? 2 * t + 1 : 2 * t + 2);
}

__global__ __launch_bounds__(kBlock) void k_tag_level(i64 n, int l, int k, const u32* __restrict__ planar0,
                                                      const u64* __restrict__ piv, u32* __restrict__ tags,
                                                      u32* __restrict__ recs) {
    const i64 stride = (i64)gridDim.x * kBlock;
    const u32 fl = (u32)full_nodes(l);
    const u64 plane = (u64)(l % k) * (u64)n, above = (u64)((l + k - 1) % k) * (u64)n;  // dimensions l, l-1
    for (i64 p = (i64)blockIdx.x * kBlock + threadIdx.x; p < n; p += stride) {
        u32 t = 0;
        if (l > 0) t = tag_descend(tags[p], planar0[above + p], (u32)p, piv);
        tags[p] = t;
        // (every record keeps its key: the first pass's digits come from it;
        // word 2 is padding, so that a record is one 16-byte access)
        reinterpret_cast<uint4*>(recs)[p] = make_uint4(planar0[plane + p], t & kFixedTag ? ~0u : t - fl, 0u, (u32)p);
    }
}

// After the last global round R-1: each point's records for the subtree
// stage, (position key, index), with the position key placing it where the
// stage looks for it, in round R-1's order of the points live on level R-1:
// node P of that level contributes its left child's points (3 (P - F(R-1))),
// its pivot (+1), then its right child's points (+2); points fixed before
// level R-1 sort last. Also the first sort pass's digit (the key's low byte).
__global__ __launch_bounds__(kBlock) void k_tag_subtrees(i64 n, int R, int k, const u32* __restrict__ planar0,
                                                         const u64* __restrict__ piv, const u32* __restrict__ tags,
                                                         u32* __restrict__ recs, u8* __restrict__ digits) {
    const i64 stride = (i64)gridDim.x * kBlock;
    const u32 fp = (u32)full_nodes(R - 1), fp1 = (u32)full_nodes(R);
    for (i64 p = (i64)blockIdx.x * kBlock + threadIdx.x; p < n; p += stride) {
        const u32 t = tag_descend(tags[p], planar0[(u64)((R - 1) % k) * (u64)n + p], (u32)p, piv);
        u32 key;
        if (t & kFixedTag) {
            const u32 node = t & ~kFixedTag;
            key = node >= fp && node < fp1 ? 3 * (node - fp) + 1 : ~0u;
        } else {
            const u32 parent = (t - 1) / 2;
            key = 3 * (parent - fp) + (t == 2 * parent + 1 ? 0u : 2u);
        }
        recs[2 * p] = key;
        recs[2 * p + 1] = (u32)p;
        digits[p] = (u8)key;
    }
}

// Split-widest rounds by per-point tags: as above, with each point's key
// read from the plane of its node's split dimension (the node table), so a
// round costs the same whatever k is; the record pass also writes the first
// sort pass's digit, the planes differing from point to point.
__global__ __launch_bounds__(kBlock) void k_wtag_level(i64 n, int l, const u32* __restrict__ planar0,
                                                       const u64* __restrict__ piv,
                                                       const uint16_t* __restrict__ dimtab, u32* __restrict__ tags,
                                                       u32* __restrict__ recs, u8* __restrict__ digits) {
    const i64 stride = (i64)gridDim.x * kBlock;
    const u32 fl = (u32)full_nodes(l);
    for (i64 p = (i64)blockIdx.x * kBlock + threadIdx.x; p < n; p += stride) {
        u32 t = 0;
        if (l > 0) {
            t = tags[p];
            if (!(t & kFixedTag)) t = tag_descend(t, planar0[(u64)dimtab[t] * (u64)n + p], (u32)p, piv);
        }
        tags[p] = t;
        const bool fixed = t & kFixedTag;
        const u32 key = planar0[(u64)(fixed ? 0u : dimtab[t]) * (u64)n + p];
        reinterpret_cast<uint4*>(recs)[p] = make_uint4(key, fixed ? ~0u : t - fl, 0u, (u32)p);
        digits[p] = (u8)key;
    }
}

// After the last global level l0 - 1 of a split-widest build: each point's
// node offset on level l0 (~0 for a fixed point) as two-word records
// (offset, index), with the first sort pass's digit.
__global__ __launch_bounds__(kBlock) void k_wtag_subtrees(i64 n, int l0, const u32* __restrict__ planar0,
                                                          const u64* __restrict__ piv,
                                                          const uint16_t* __restrict__ dimtab,
                                                          const u32* __restrict__ tags, u32* __restrict__ recs,
                                                          u8* __restrict__ digits) {
    const i64 stride = (i64)gridDim.x * kBlock;
    const u32 fl = (u32)full_nodes(l0);
    for (i64 p = (i64)blockIdx.x * kBlock + threadIdx.x; p < n; p += stride) {
        u32 t = tags[p];
        if (!(t & kFixedTag)) t = tag_descend(t, planar0[(u64)dimtab[t] * (u64)n + p], (u32)p, piv);
        const u32 off = t & kFixedTag ? ~0u : t - fl;
        reinterpret_cast<uint2*>(recs)[p] = make_uint2(off, (u32)p);
        digits[p] = (u8)off;
    }
}

// The subtree stage's planar records (k keys, then the index) of the points
// live on level l0, in their sorted order (subtree by subtree, each in index
// order), from each point's row.
__global__ __launch_bounds__(kBlock) void k_wtag_planar(i64 live, i64 n, int k, const float* __restrict__ pts,
                                                        const u32* __restrict__ sorted, u32* __restrict__ out) {
    const i64 stride = (i64)gridDim.x * kBlock;
    for (i64 q = (i64)blockIdx.x * kBlock + threadIdx.x; q < live; q += stride) {
        const u32 idx = sorted[2 * q + 1];
        const u32* row = reinterpret_cast<const u32*>(pts) + (u64)idx * k;
        for (int d = 0; d < k; ++d) out[(u64)d * (u64)n + q] = float_key(row[d]);
        out[(u64)k * (u64)n + q] = idx;
    }
}

// Tags after `rounds` rounds by walking the pivots from the root (the node
// the point reaches, or the node it became): diagnostics only.
__global__ __launch_bounds__(kBlock) void k_descend_tags(const float* __restrict__ pts, i64 n,
                                                         int k, int rounds,
                                                         const u64* __restrict__ piv,
                                                         u32* __restrict__ tags) {
    const i64 stride = (i64)gridDim.x * kBlock;
    for (i64 i = (i64)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        u64 s = 0;
        int dim = 0;
        for (int l = 0; l < rounds; ++l) {
            const u64 me = ((u64)float_key(__float_as_uint(pts[i * k + dim])) << 32) | (u64)i;
            const u64 p = piv[s];
            if (me == p) break;
            s = me < p ? 2 * s + 1 : 2 * s + 2;
            if (++dim == k) dim = 0;
        }
        tags[i] = (u32)s;
    }
}

// ------------------------------------ split-widest-dimension domains
// [W], split-widest-dimension section: the root's domain is the bounding box
// of all points; every node splits the dimension in which its domain is
// widest (float32 extent hi - lo, the lower dimension on ties); a child's
// domain is its parent's, bounded at the parent's plane (its point's
// coordinate in the parent's dimension: upper bound for the left child,
// lower bound for the right one).

// Per-dimension minimum and maximum of one chunk of points (grid: chunks x
// k); partial[(d * chunks + c) * 2 + {0, 1}].
__global__ __launch_bounds__(kBlock) void k_box_partial(const float* __restrict__ pts, i64 n, int k,
                                                        i64 chunk, float* __restrict__ partial) {
    const int d = blockIdx.y;
    const i64 c = blockIdx.x, first = c * chunk;
    const i64 last = first + chunk < n ? first + chunk : n;
    float lo = __uint_as_float(0x7f800000u), hi = __uint_as_float(0xff800000u);  // +inf, -inf
    for (i64 i = first + threadIdx.x; i < last; i += kBlock) {
        const float x = pts[i * k + d];
        if (x < lo) lo = x;
        if (hi < x) hi = x;
    }
    __shared__ float s_lo[kWaves], s_hi[kWaves];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ol = __shfl_xor(lo, o, 64), oh = __shfl_xor(hi, o, 64);
        if (ol < lo) lo = ol;
        if (hi < oh) hi = oh;
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_lo[w] = lo;
        s_hi[w] = hi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int v = 1; v < kWaves; ++v) {
            if (s_lo[v] < lo) lo = s_lo[v];
            if (hi < s_hi[v]) hi = s_hi[v];
        }
        partial[(d * (i64)gridDim.x + c) * 2] = lo;
        partial[(d * (i64)gridDim.x + c) * 2 + 1] = hi;
    }
}

// The same for k <= 4 and 16-byte-aligned rows, every dimension in one
// pass: a thread reads four points at a time as kK 16-byte words (float f
// of the four is coordinate f mod kK of point f / kK).
template <int kK>
__global__ __launch_bounds__(kBlock) void k_box_partial4(const float* __restrict__ pts, i64 n, i64 chunk,
                                                         float* __restrict__ partial) {
    const i64 c = blockIdx.x, first = c * chunk;  // (chunk is a multiple of 4)
    const i64 last = first + chunk < n ? first + chunk : n;
    float lo[kK], hi[kK];
#pragma unroll
    for (int d = 0; d < kK; ++d) {
        lo[d] = __uint_as_float(0x7f800000u);
        hi[d] = __uint_as_float(0xff800000u);
    }
    const float4* quads = reinterpret_cast<const float4*>(pts);
    for (i64 g = first / 4 + threadIdx.x; g < last / 4; g += kBlock) {
        float4 w[kK];
#pragma unroll
        for (int q = 0; q < kK; ++q) w[q] = quads[g * kK + q];
#pragma unroll
        for (int f = 0; f < 4 * kK; ++f) {
            const float4 v = w[f / 4];
            const float x = f % 4 == 0 ? v.x : f % 4 == 1 ? v.y : f % 4 == 2 ? v.z : v.w;
            if (x < lo[f % kK]) lo[f % kK] = x;
            if (hi[f % kK] < x) hi[f % kK] = x;
        }
    }
    for (i64 i = last / 4 * 4 + threadIdx.x; i < last; i += kBlock)  // the last chunk's tail
#pragma unroll
        for (int d = 0; d < kK; ++d) {
            const float x = pts[i * kK + d];
            if (x < lo[d]) lo[d] = x;
            if (hi[d] < x) hi[d] = x;
        }
    __shared__ float s_lo[kK][kWaves], s_hi[kK][kWaves];
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int d = 0; d < kK; ++d) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ol = __shfl_xor(lo[d], o, 64), oh = __shfl_xor(hi[d], o, 64);
            if (ol < lo[d]) lo[d] = ol;
            if (hi[d] < oh) hi[d] = oh;
        }
        if ((threadIdx.x & 63) == 0) {
            s_lo[d][w] = lo[d];
            s_hi[d][w] = hi[d];
        }
    }
    __syncthreads();
    if (threadIdx.x < kK) {
        const int d = threadIdx.x;
        float l = s_lo[d][0], h = s_hi[d][0];
        for (int v = 1; v < kWaves; ++v) {
            if (s_lo[d][v] < l) l = s_lo[d][v];
            if (h < s_hi[d][v]) h = s_hi[d][v];
        }
        partial[(d * (i64)gridDim.x + c) * 2] = l;
        partial[(d * (i64)gridDim.x + c) * 2 + 1] = h;
    }
}

// The root domain (lo[0..k), hi[0..k)) from the chunks' (grid: k blocks).
__global__ __launch_bounds__(kBlock) void k_box_final(const float* __restrict__ partial, i64 chunks,
                                                      int k, float* __restrict__ box) {
    const int d = blockIdx.x;
    float lo = __uint_as_float(0x7f800000u), hi = __uint_as_float(0xff800000u);
    for (i64 c = threadIdx.x; c < chunks; c += kBlock) {
        const float pl = partial[(d * chunks + c) * 2], ph = partial[(d * chunks + c) * 2 + 1];
        if (pl < lo) lo = pl;
        if (hi < ph) hi = ph;
    }
    __shared__ float s_lo[kWaves], s_hi[kWaves];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ol = __shfl_xor(lo, o, 64), oh = __shfl_xor(hi, o, 64);
        if (ol < lo) lo = ol;
        if (hi < oh) hi = oh;
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_lo[w] = lo;
        s_hi[w] = hi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int v = 1; v < kWaves; ++v) {
            if (s_lo[v] < lo) lo = s_lo[v];
            if (hi < s_hi[v]) hi = s_hi[v];
        }
        box[d] = lo;
        box[k + d] = hi;
    }
}

// A child's domain (2k floats: lo then hi) from its parent's domain `from`,
// bounded at `plane` in the parent's dimension pd (pd < 0: the domain
// itself); returns the dimension of its widest extent.
__device__ __forceinline__ int child_domain(const float* from, int pd, float plane, bool left, int k,
                                            float* box) {
    int best = 0;
    float best_extent = 0.0f;
    for (int d = 0; d < k; ++d) {
        float lo = from[d], hi = from[k + d];
        if (d == pd) {
            if (left) hi = plane;
            else lo = plane;
        }
        box[d] = lo;
        box[k + d] = hi;
        const float extent = hi - lo;
        if (d == 0) best_extent = extent;
        else if (extent > best_extent) {
            best = d;
            best_extent = extent;
        }
    }
    return best;
}

// Domains and split dimensions of the nodes of level l (2k floats a node:
// lo then hi), from their parents' (the root's from the bounding box). The
// parents' pivots are fixed.
// level_dims (k <= 32, else nullptr): bit d of level_dims[l] is set when
// some node of level l splits dimension d.
__global__ __launch_bounds__(kBlock) void k_widest_level(Geometry geo, int l, int k,
                                                         const u64* __restrict__ piv,
                                                         const float* __restrict__ root_box,
                                                         float* __restrict__ boxes,
                                                         uint16_t* __restrict__ dimtab,
                                                         int32_t* __restrict__ dims_out,
                                                         u32* __restrict__ level_dims) {
    const u64 j = (u64)blockIdx.x * kBlock + threadIdx.x;
    const u64 s = full_nodes(l) + j;
    const bool here = j < (1ull << l) && s < (u64)geo.n;
    u32 bits = 0;
    if (here) {
        const float* from = root_box;
        int pd = -1;
        float plane = 0.0f;
        bool left = false;
        if (l > 0) {
            const u64 p = (s - 1) / 2;
            from = boxes + p * 2 * (u64)k;
            pd = dimtab[p];
            plane = __uint_as_float(key_bits((u32)(piv[p] >> 32)));  // a zero's sign is lost: extents agree
            left = s == 2 * p + 1;
        }
        const int best = child_domain(from, pd, plane, left, k, boxes + s * 2 * (u64)k);
        dimtab[s] = (uint16_t)best;
        if (dims_out) dims_out[s] = best;
        bits = best < 32 ? 1u << best : 0u;
    }
    if (level_dims) {  // one atomic per wave: the OR of its nodes' bits
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) bits |= __shfl_xor(bits, o, 64);
        if ((threadIdx.x & 63) == 0 && bits) atomicOr(&level_dims[l], bits);
    }
}

// ------------------------------------------------- duplicate removal
// [R], duplicate-removal section: with the tuples sorted by all their
// coordinates, equal tuples are adjacent and all but one of each run go. Here
// the records are sorted by the keys of coordinates 0 .. k-1 (coordinate 0
// most significant) and then by index, so the first record of a run has the
// group's smallest index; its index is flagged, and a compaction in index
// order lists the kept indices ascending.

constexpr int kFlagItems = 16;                  // flags per thread (one 16-byte load)
constexpr int kFlagTile = kBlock * kFlagItems;  // flags per compaction workgroup

// keep[idx] = 1 for the first record of every run of equal tuples, else 0.
// Equal tuples hash equally: MurmurHash3's 32-bit finaliser chained over the
// coordinate keys (zeros canonical, so -0.0 and +0.0 agree).
__device__ __forceinline__ u32 fmix32(u32 h) {
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

__device__ __forceinline__ u32 tuple_hash(const float* __restrict__ pts, int k, i64 i) {
    u32 h = 0x9e3779b9u;
    for (int d = 0; d < k; ++d) h = fmix32(h ^ float_key(__float_as_uint(pts[i * k + d])));
    return h;
}

// Records (hash, index) in index order, and the low hash byte (the first
// sort pass's digit).
__global__ __launch_bounds__(kBlock) void k_hash_records(const float* __restrict__ pts, i64 n, int k,
                                                         u32* __restrict__ recs, u8* __restrict__ digits) {
    const i64 stride = (i64)gridDim.x * kBlock;
    for (i64 i = (i64)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        const u32 h = tuple_hash(pts, k, i);
        *reinterpret_cast<uint2*>(recs + 2 * i) = make_uint2(h, (u32)i);
        digits[i] = (u8)h;
    }
}

// Whether points a and b are the same tuple (keys: equal iff the floats are).
__device__ __forceinline__ bool same_tuple(const float* __restrict__ pts, int k, u32 a, u32 b) {
    for (int d = 0; d < k; ++d)
        if (float_key(__float_as_uint(pts[(i64)a * k + d])) != float_key(__float_as_uint(pts[(i64)b * k + d])))
            return false;
    return true;
}

// keep[0 .. n) = 1, a 32-bit word at a time (the buffer is padded to 4).
__global__ __launch_bounds__(kBlock) void k_keep_all(u32* __restrict__ keep_words, i64 words) {
    const i64 stride = (i64)gridDim.x * kBlock;
    for (i64 i = (i64)blockIdx.x * kBlock + threadIdx.x; i < words; i += stride) keep_words[i] = 0x01010101u;
}

// Run heads of the records sorted by (hash, index): a point is kept when no
// earlier record of its equal-hash run (a smaller index) holds the same
// tuple. The scan back stops at the first equal tuple, so a run of copies
// costs one comparison per record; only distinct tuples that share a hash
// compare further. keep[index] = 0 for the points that are not kept (keep
// starts all ones), so only duplicates cost a scattered store.
__global__ __launch_bounds__(kBlock) void k_unique_mark(const u32* __restrict__ recs, i64 n,
                                                        const float* __restrict__ pts, int k,
                                                        u8* __restrict__ keep) {
    const i64 stride = (i64)gridDim.x * kBlock;
    for (i64 r = (i64)blockIdx.x * kBlock + threadIdx.x; r < n; r += stride) {
        const uint2 me = *reinterpret_cast<const uint2*>(recs + 2 * r);
        bool head = true;
        for (i64 p = r - 1; p >= 0 && recs[2 * p] == me.x; --p)
            if (same_tuple(pts, k, me.y, recs[2 * p + 1])) {
                head = false;
                break;
            }
        if (!head) keep[me.y] = 0;
    }
}

// The kFlagItems flags of this thread (0 past n).
__device__ inline void load_flags(const u8* keep, i64 n, i64 first, u32 (&w)[4]) {
    if (first + kFlagItems <= n) {
        const uint4 v = *reinterpret_cast<const uint4*>(keep + first);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
    } else {
        w[0] = w[1] = w[2] = w[3] = 0;
        for (int j = 0; j < kFlagItems; ++j)
            if (first + j < n) w[j >> 2] |= (u32)keep[first + j] << (8 * (j & 3));
    }
}

// Kept indices per tile of kFlagTile flags.
__global__ __launch_bounds__(kBlock) void k_flag_count(const u8* __restrict__ keep, i64 n,
                                                       u32* __restrict__ counts) {
    __shared__ u32 s_wave[kWaves];
    const i64 first = (i64)blockIdx.x * kFlagTile + (i64)threadIdx.x * kFlagItems;
    u32 w[4];
    load_flags(keep, n, first, w);
    const u32 mine = __popc(w[0]) + __popc(w[1]) + __popc(w[2]) + __popc(w[3]);  // flags are 0 or 1
    const u32 before = block_exclusive_scan(mine, s_wave);
    if (threadIdx.x == kBlock - 1) counts[blockIdx.x] = before + mine;
}

// Writes the kept indices of one tile at their places (prefix: kept indices
// in the tiles before, from k_chunk_scan), and the total to *count_out. The
// tile's kept indices are gathered in LDS first, so that consecutive
// threads write consecutive entries.
__global__ __launch_bounds__(kBlock) void k_flag_compact(const u8* __restrict__ keep, i64 n,
                                                         const u32* __restrict__ prefix,
                                                         const u32* __restrict__ totals,
                                                         int32_t* __restrict__ keep_out,
                                                         int64_t* __restrict__ count_out) {
    __shared__ u32 s_wave[kWaves];
    __shared__ int32_t s_kept[kFlagTile];
    __shared__ u32 s_total;
    const i64 first = (i64)blockIdx.x * kFlagTile + (i64)threadIdx.x * kFlagItems;
    u32 w[4];
    load_flags(keep, n, first, w);
    const u32 mine = __popc(w[0]) + __popc(w[1]) + __popc(w[2]) + __popc(w[3]);
    u32 at = block_exclusive_scan(mine, s_wave);
    if (threadIdx.x == kBlock - 1) s_total = at + mine;
#pragma unroll
    for (int j = 0; j < kFlagItems; ++j)
        if ((w[j >> 2] >> (8 * (j & 3))) & 1u) s_kept[at++] = (int32_t)(first + j);
    __syncthreads();
    const u32 base = prefix[blockIdx.x], total = s_total;
    for (u32 i = threadIdx.x; i < total; i += kBlock) keep_out[base + i] = s_kept[i];
    if (blockIdx.x == 0 && threadIdx.x == 0) *count_out = (int64_t)totals[0];
}

__global__ __launch_bounds__(kBlock) void k_zero(u32* __restrict__ out, i64 n) {
    const i64 stride = (i64)gridDim.x * kBlock;
    for (i64 e = (i64)blockIdx.x * kBlock + threadIdx.x; e < n; e += stride) out[e] = 0u;
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
static_assert(kLocalBlock >= kRadix, "one thread per digit");

// x, which the compiler can neither fold nor hoist out of a loop: keeps a
// cheap per-lane value from being held (or spilled) across a long loop.
__device__ __forceinline__ u32 opaque(u32 x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Slot of item j of this thread: each wave owns kLocalItems rows of 64.
__device__ inline int local_slot(int j) {
    return (threadIdx.x >> 6) * (64 * kLocalItems) + j * 64 + (threadIdx.x & 63);
}

struct SubtreeArgs {
    const float* pts;
    i64 n;
    int k;
    int l0;                 // level of the subtree roots
    Geometry geo;
    const u32* recs;        // l0 > 0: records (coordinates 0 .. words-2, then the
    int words;              // index) live on level l0-1, in round l0-1's order
    u64 plane;              // their plane stride (records wider than kWholeWords)
    bool index_only;        // the records' last word is the index and they carry no
                            // coordinate; each subtree's arrive in index order
    u32* stage;             // 1 + min(k, kLocalRounds) columns of n words: the index, then
                            // the key column of each dimension the local rounds split, by
                            // round (dimension (l0 + u) mod k in column u + 1); the subtree
                            // owns [first, first + |S(c)|) of each
    int32_t* perm;
    float* tree;
};

// ------------------------- subtree stage from records with every coordinate
// The subtree stage for k <= kCachedDims, where the records of the last
// global round carry all k coordinate keys: the same rounds as k_subtree_cols,
// organised so that each record is read once as one vector, and every radix
// pass in LDS moves one 32-bit word per point. A pass sorts a value stably:
// the value less its minimum over the subtree, so that only the bits in which
// the subtree's values differ are sorted (for a level-12 subtree of the
// headline workload about 19 bits of a coordinate key), in passes of at most
// 8 bits; as soon as the unsorted rest fits 20 bits it travels together with
// a 12-bit payload (the point's arrival position or slot) in one word.
// Positions past the subtree's size hold padding that sorts last and whose
// tag is never live, so no per-item loop tests for them.
constexpr int kPay = 12;  // bits of a slot or an arrival position
static_assert(kLocalMax <= (1 << kPay), "a slot fits the payload");
constexpr u32 kPadTag = 0xffffu;  // tag of a padding slot: never on a level

struct RecScratch {
    u32 exch[2][kLocalMax];                // record exchange; the rounds' segment counters
    uint16_t count[kLocalWaves][kRadix];   // per-wave digit counters of a pass
    u32 start[kRadix];                     // first position of each digit
    u32 wave[kLocalWaves];
    u32 red[2 * (kCachedDims + 1)][kLocalWaves];  // per-wave minima and maxima
    uint16_t dummy[64];                    // counter of the items a round does not rank
};

struct RecShared {
    union {
        struct {
            uint16_t tag[kLocalMax];                 // local tag of each slot
            uint16_t order[kCachedDims][kLocalMax];  // slots by (coordinate d, index)
            RecScratch s;
        } m;
        uint4 rows[kLocalMax];  // output: the record of each local node
    };
};

// Lanes below this one in a 64-bit lane mask.
__device__ __forceinline__ u32 lanes_below(u32 m_lo, u32 m_hi) {
    return __builtin_amdgcn_mbcnt_hi(m_hi, __builtin_amdgcn_mbcnt_lo(m_lo, 0u));
}

// The lanes of `within` (a lane mask) whose low `bits` bits of d equal this
// lane's: per bit, the lanes whose bit agrees with this lane's are NOT(vote
// ^ own-bit-mask); the AND over the bits is kept with one three-input bit
// operation per half (truth table 0x90 over (mask, vote, m): mask & ~(vote ^
// m)), so no mask needs inverting or clearing.
__device__ __forceinline__ void peer_mask(u32 d, int bits, u32 within_lo, u32 within_hi, u32& p_lo,
                                          u32& p_hi) {
    p_lo = within_lo;
    p_hi = within_hi;
    for (int b = 0; b < bits; ++b) {
        u32 m = (u32)__builtin_amdgcn_sbfe((int)d, b, 1);
        // (opaque, so that the vote compares m itself rather than testing the
        // bit of d again with a shift of its own: one VALU instruction less)
        asm("" : "+v"(m));
        const u64 vote = __ballot(m != 0);
        p_lo = __builtin_amdgcn_bitop3_b32(p_lo, (u32)vote, m, 0x90);
        p_hi = __builtin_amdgcn_bitop3_b32(p_hi, (u32)(vote >> 32), m, 0x90);
    }
}

// One stable pass by the low `bits` bits of each item's unsorted value.
// Wide form: hi = the value, lo = the payload. Narrow form: hi = value << kPay
// | payload. The pass drops the sorted bits; kWideOut keeps the wide form
// (the rest does not fit 32 - kPay bits yet), its payloads exchanged through
// pay_x (kLocalMax 16-bit entries). S is the scratch type (RecScratch or
// ColScratch): only its first exchange buffer is used.
// kBits > 0: the digit width as a compile-time constant (bits_rt unused), so
// that the ballot match unrolls.
template <bool kWideIn, bool kWideOut, int kBits, typename S>
__device__ __forceinline__ void rec_pass(u32 (&hi)[kLocalItems], u32 (&lo)[kLocalItems], int bits_rt, S& s,
                                         uint16_t* pay_x) {
    const int bits = kBits > 0 ? kBits : bits_rt;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const u32 bins = 1u << bits;
    uint16_t* cnt = s.count[w];
    // (cleared through the same type the ranking reads: no barrier between)
    for (u32 i = lane; i < bins; i += 64) cnt[i] = 0;
    auto digit = [&](int j) { return __builtin_amdgcn_ubfe(hi[j], kWideIn ? 0 : kPay, bits); };
    u32 rank[kLocalItems];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 d = digit(j);
        u32 p_lo, p_hi;
        peer_mask(d, bits, ~0u, ~0u, p_lo, p_hi);
        const u32 before = lanes_below(p_lo, p_hi);
        const u32 seen = cnt[d];
        rank[j] = seen + before;
        // every lane of the digit writes the same count
        cnt[d] = (uint16_t)(seen + __popc(p_lo) + __popc(p_hi));
    }
    __syncthreads();
    // per digit: prefix over the waves, then the exclusive scan of the totals
    u32 agg = 0;
    if ((u32)tid < bins) {
#pragma unroll
        for (int v = 0; v < kLocalWaves; ++v) {
            const u32 c = s.count[v][tid];
            s.count[v][tid] = (uint16_t)agg;
            agg += c;
        }
    }
    const u32 inc = wave_inclusive_scan(agg);
    if (lane == 63) s.wave[w] = inc;
    __syncthreads();
    if ((u32)tid < bins) {
        u32 off = 0;
#pragma unroll
        for (int i = 0; i < kLocalWaves; ++i)
            if (i < w) off += s.wave[i];
        s.start[tid] = off + inc - agg;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {  // all reads before the exchange writes
        const u32 d = digit(j);
        rank[j] += s.start[d] + s.count[w][d];
    }
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 pos = rank[j];
        if constexpr (kWideOut) {
            s.exch[0][pos] = hi[j] >> bits;
            pay_x[pos] = (uint16_t)lo[j];
        } else {
            const u32 rest = kWideIn ? hi[j] >> bits : hi[j] >> (kPay + bits);
            const u32 pay = kWideIn ? lo[j] : hi[j] & ((1u << kPay) - 1);
            s.exch[0][pos] = (rest << kPay) | pay;
        }
    }
    __syncthreads();
    // (the next pass's first barrier orders these reads before its writes)
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const int q = local_slot(j);
        hi[j] = s.exch[0][q];
        if constexpr (kWideOut) lo[j] = pay_x[q];
    }
}

// A pass of the common digit widths (6 to 8 bits) with its match unrolled.
template <bool kWideIn, bool kWideOut, typename S>
__device__ __forceinline__ void rec_pass_any(u32 (&hi)[kLocalItems], u32 (&lo)[kLocalItems], int bits, S& s,
                                             uint16_t* pay_x) {
    if (bits == 8) rec_pass<kWideIn, kWideOut, 8>(hi, lo, bits, s, pay_x);
    else if (bits == 7) rec_pass<kWideIn, kWideOut, 7>(hi, lo, bits, s, pay_x);
    else if (bits == 6) rec_pass<kWideIn, kWideOut, 6>(hi, lo, bits, s, pay_x);
    else rec_pass<kWideIn, kWideOut, 0>(hi, lo, bits, s, pay_x);
}

// Stable sort of the items (value v[j] below 2^vbits, payload pay[j] below
// 2^kPay) from their current order; returns with pay[j] = the payload of the
// item at position local_slot(j). vbits = 0: nothing to sort. pay_x as in
// rec_pass (RecScratch: its second exchange buffer).
template <typename S>
__device__ __forceinline__ void rec_sort(u32 (&v)[kLocalItems], u32 (&pay)[kLocalItems], int vbits, S& s,
                                         uint16_t* pay_x) {
    if (vbits == 0) return;
    const int passes = (vbits + kRadixBits - 1) / kRadixBits;
    int left = vbits;
    bool wide = true;
    for (int p = 0; p < passes; ++p) {
        const int bits = (left + (passes - p) - 1) / (passes - p);
        const bool out_wide = left - bits > 32 - kPay;
        if (wide && out_wide) rec_pass_any<true, true>(v, pay, bits, s, pay_x);
        else if (wide) rec_pass_any<true, false>(v, pay, bits, s, pay_x);
        else rec_pass_any<false, false>(v, pay, bits, s, pay_x);
        wide = out_wide;
        left -= bits;
    }
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) pay[j] = v[j] & ((1u << kPay) - 1);
}

__device__ __forceinline__ void rec_sort(u32 (&v)[kLocalItems], u32 (&pay)[kLocalItems], int vbits,
                                         RecScratch& s) {
    rec_sort(v, pay, vbits, s, reinterpret_cast<uint16_t*>(&s.exch[1][0]));
}

// Workgroup minimum and maximum of each of kV values, from each thread's own.
template <int kV, typename S>
__device__ __forceinline__ void rec_min_max(u32 (&mn)[kV], u32 (&mx)[kV], S& s) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kV; ++i) {
        u32 a = mn[i], b = mx[i];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const u32 oa = __shfl_xor(a, o, 64), ob = __shfl_xor(b, o, 64);
            a = oa < a ? oa : a;
            b = ob > b ? ob : b;
        }
        if (lane == 0) {
            s.red[2 * i][w] = a;
            s.red[2 * i + 1][w] = b;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kV; ++i) {
        u32 a = ~0u, b = 0;
#pragma unroll
        for (int v = 0; v < kLocalWaves; ++v) {
            a = s.red[2 * i][v] < a ? s.red[2 * i][v] : a;
            b = s.red[2 * i + 1][v] > b ? s.red[2 * i + 1][v] : b;
        }
        // uniform over the workgroup: scalar registers
        mn[i] = __builtin_amdgcn_readfirstlane(a);
        mx[i] = __builtin_amdgcn_readfirstlane(b);
    }
}

// Bits that values 0 .. span (and the padding value above them) need.
__device__ __forceinline__ int value_bits(u32 span) { return span == ~0u ? 32 : 32 - __clz(span + 1); }

// Round t in LDS. A segment's sorted position is its closed-form start plus
// a point's rank among the segment's points earlier in `order` (slots by
// (coordinate, index)); that rank is all the round needs, so no record
// moves. It is counted per wave by ballots over the 2^t live segments, then
// prefixed across waves, and compared with the left subtree's size: below,
// the point goes to the left child, above to the right one, equal it is the
// node. Padding slots carry kPadTag: per-wave counters of the 2^t segments live in the exchange
// buffers from the first on (Count: 16-bit, 8 x 2048 of them spanning both
// of RecScratch's; 8-bit where a segment holds at most 255 points); items
// that are not live count into a dummy and write their tag back unchanged.
// With nodedim (split-widest trees), only the segments whose node splits
// dimension d are live.
// kT >= 0: the round index as a compile-time constant (t_rt unused), so that
// the t-bit ballot match unrolls.
template <int kT, typename Count, typename S>
__device__ __forceinline__ void rec_round_at(const uint16_t* order, int t_rt, const Geometry& lg, uint16_t* tag,
                                             S& s, const uint8_t* nodedim, u32 d) {
    const int t = kT >= 0 ? kT : t_rt;
    // (thread-derived offsets recomputed a call, not held across the level loop)
    const int tid = (int)opaque(threadIdx.x), lane = tid & 63, w = tid >> 6;
    const u32 fl = (1u << t) - 1, segs = 1u << t;
    Count* cnt = reinterpret_cast<Count*>(&s.exch[0][0]);  // [kLocalWaves][segs]
    u32* cnt_words = &s.exch[0][0];
    const u32 words = (kLocalWaves * segs * (u32)sizeof(Count) + 3) / 4;
    for (u32 i = tid; i < words; i += kLocalBlock) cnt_words[i] = 0;
    __syncthreads();
    // Every item's slot and tag first: reads issued back to back (the
    // counter writes below could alias them, so they would otherwise wait
    // for each other item by item).
    u32 e[kLocalItems], st[kLocalItems], rank[kLocalItems];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) e[j] = order[local_slot(j)];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) st[j] = tag[e[j]];
    // (a padding tag is never below fl + segs, so nodedim is read in range)
    bool on[kLocalItems];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        on[j] = st[j] - fl < segs;
        if (nodedim && on[j]) on[j] = nodedim[st[j]] == d;
    }
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 b = st[j] - fl;
        const bool live = on[j];
        const u64 lv = __ballot(live);
        u32 p_lo, p_hi;
        peer_mask(b, t, (u32)lv, (u32)(lv >> 32), p_lo, p_hi);
        const u32 before = lanes_below(p_lo, p_hi);
        Count* cp = live ? &cnt[w * segs + b] : reinterpret_cast<Count*>(s.dummy) + lane;
        const u32 seen = *cp;
        rank[j] = seen + before;
        *cp = (Count)(seen + __popc(p_lo) + __popc(p_hi));
    }
    __syncthreads();
    // prefix over the waves, a word of counters at a time (a segment's total
    // fits its counter, so the counters of a word never carry into each other)
    if (segs * sizeof(Count) >= 4) {
        const u32 row = segs * (u32)sizeof(Count) / 4;
        for (u32 i = tid; i < row; i += kLocalBlock) {
            u32 run = 0;
#pragma unroll
            for (int v = 0; v < kLocalWaves; ++v) {
                const u32 c = cnt_words[v * row + i];
                cnt_words[v * row + i] = run;
                run += c;
            }
        }
    } else if ((u32)tid < segs) {
        u32 run = 0;
#pragma unroll
        for (int v = 0; v < kLocalWaves; ++v) {
            const u32 c = cnt[v * segs + tid];
            cnt[v * segs + tid] = (Count)run;
            run += c;
        }
    }
    __syncthreads();
    // the pivot of segment s = F(t) + b has rank |S(2s+1)|: u - 1 full-level
    // nodes and min(max(M - 2b u, 0), u) last-level ones (u = 2^(L-2-t))
    const u32 dd = (u32)(lg.levels - 2 - t), u = 1u << dd, last = (u32)lg.last;
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 b = st[j] - fl;
        rank[j] += cnt[w * segs + (b < segs ? b : 0)];  // all reads before the tag writes
    }
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 b = st[j] - fl;
        const bool live = on[j];
        const u32 in_seg = rank[j];
        const u32 under = (2 * b) << dd;
        const u32 left = (u - 1) + (last > under ? (last - under < u ? last - under : u) : 0u);
        const u32 next = in_seg < left ? 2 * st[j] + 1 : (in_seg > left ? 2 * st[j] + 2 : st[j]);
        tag[e[j]] = (uint16_t)(live ? next : st[j]);
    }
    __syncthreads();
}

template <typename Count = uint16_t, typename S>
__device__ __forceinline__ void rec_round(const uint16_t* order, int t, const Geometry& lg, uint16_t* tag,
                                          S& s, const uint8_t* nodedim = nullptr, u32 d = 0) {
    switch (t) {  // every round of a kLocalMax-point subtree: t <= kLocalRounds - 1
#define KDT_ROUND_CASE(T) \
    case T: rec_round_at<T, Count>(order, t, lg, tag, s, nodedim, d); break;
        KDT_ROUND_CASE(0) KDT_ROUND_CASE(1) KDT_ROUND_CASE(2) KDT_ROUND_CASE(3)
        KDT_ROUND_CASE(4) KDT_ROUND_CASE(5) KDT_ROUND_CASE(6) KDT_ROUND_CASE(7)
        KDT_ROUND_CASE(8) KDT_ROUND_CASE(9) KDT_ROUND_CASE(10) KDT_ROUND_CASE(11)
#undef KDT_ROUND_CASE
        default: rec_round_at<-1, Count>(order, t, lg, tag, s, nodedim, d); break;
    }
}

template <int kK>
__global__ __launch_bounds__(kLocalBlock, 4) void k_subtree_recs(SubtreeArgs a) {
    static_assert(kK >= 1 && kK <= kCachedDims, "every coordinate in the record");
    constexpr int kW = kK + 1;  // record words: the keys, then the index
    __shared__ RecShared sh;
    RecScratch& s = sh.m.s;

    const u64 c = full_nodes(a.l0) + blockIdx.x;  // subtree root (global node id)
    const u32 nc = (u32)subtree_size(a.geo, c);
    if (nc == 0) return;
    // live position of the subtree's first point in round l0-1's order
    const u64 parent = (c - 1) / 2;
    const u64 seg = live_begin(a.geo, parent - full_nodes(a.l0 - 1), a.l0 - 1);
    const u64 first = c == 2 * parent + 1 ? seg : seg + subtree_size(a.geo, 2 * parent + 1) + 1;
    const u32* recs = a.recs + first * kW;
    auto load_record = [&](u32 q, u32 (&r)[kW]) {
        const u32* src = recs + (u64)(q < nc ? q : nc - 1) * kW;
        if constexpr (kW == 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(src);
            r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
        } else if constexpr (kW == 2) {
            const uint2 v = *reinterpret_cast<const uint2*>(src);
            r[0] = v.x; r[1] = v.y;
        } else {
#pragma unroll
            for (int f = 0; f < kW; ++f) r[f] = src[f];
        }
    };

    // Word f of a record held as four registers (f uniform: selects, so that
    // no register array is indexed at run time).
    auto pick = [](const u32 (&r)[4], int f) {
        return f == 0 ? r[0] : f == 1 ? r[1] : f == 2 ? r[2] : r[3];
    };
    // Dimensions: d_a arrived sorted (round l0-1's order: by coordinate d_a,
    // then index); dA = d_a + 1 and dB = d_a + 2 (mod k), as far as k has
    // them, are sorted here.
    const int d_a = (a.l0 - 1) % kK;
    const int dA = (d_a + 1) % kK, dB = (d_a + 2) % kK;
    constexpr int kOther = kK - 1;
    // While the slots are sorted, the tags and orders are unused: the other
    // dimensions' keys wait there by arrival position.
    u32* stash = reinterpret_cast<u32*>(&sh.m.tag[0]);
    static_assert(sizeof(sh.m.tag) + sizeof(sh.m.order) >= 2 * kLocalMax * sizeof(u32), "stash");

    // The records in arrival order, one vector load each: index and the
    // other keys; minima and maxima over the subtree's points.
    u32 idx[kLocalItems];
    u32 mn[1 + kOther], mx[1 + kOther];
#pragma unroll
    for (int i = 0; i <= kOther; ++i) {
        mn[i] = ~0u;
        mx[i] = 0;
    }
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 q = (u32)local_slot(j);
        u32 r[4] = {0, 0, 0, 0};
        load_record(q, reinterpret_cast<u32(&)[kW]>(r));
        const bool ok = q < nc;
        idx[j] = r[kK];
        mn[0] = ok && idx[j] < mn[0] ? idx[j] : mn[0];
        mx[0] = ok && idx[j] > mx[0] ? idx[j] : mx[0];
#pragma unroll
        for (int u = 0; u < kOther; ++u) {
            const u32 key = pick(r, u == 0 ? dA : dB);
            stash[u * kLocalMax + q] = key;
            mn[1 + u] = ok && key < mn[1 + u] ? key : mn[1 + u];
            mx[1 + u] = ok && key > mx[1 + u] ? key : mx[1 + u];
        }
    }
    rec_min_max<1 + kOther>(mn, mx, s);
    int vbits[1 + kOther];
    u32 pad[1 + kOther];
#pragma unroll
    for (int i = 0; i <= kOther; ++i) {
        vbits[i] = value_bits(mx[i] - mn[i]);
        pad[i] = vbits[i] == 32 ? ~0u : (1u << vbits[i]) - 1;  // above every point's value
    }

    // Slot = index rank: sort (index - min, arrival position).
    u32 arr[kLocalItems];  // arrival position of the point in slot local_slot(j)
    {
        u32 v[kLocalItems];
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const u32 q = (u32)local_slot(j);
            v[j] = q < nc ? idx[j] - mn[0] : pad[0];
            arr[j] = q;
        }
        rec_sort(v, arr, vbits[0], s);
    }
    // The other dimensions' keys by slot, straight from the stash; the second
    // one waits in LDS again (by slot) while the first is sorted.
    u32 key[kLocalItems], key2[kLocalItems];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const bool ok = (u32)local_slot(j) < nc;
        if constexpr (kOther > 0) key[j] = ok ? stash[arr[j]] - mn[1] : pad[1];
        if constexpr (kOther > 1) key2[j] = ok ? stash[kLocalMax + arr[j]] - mn[2] : pad[2];
    }
    __syncthreads();  // stash read before the tags and orders overwrite it
    // Orders by role: [0] dimension d_a, [1] dA, [2] dB. The arrival order is
    // d_a's: order[0][q] = slot of arrival position q (padding positions map
    // to padding slots). dB's keys wait in roles 1 and 2 (one 16 KB range).
    u32* wait2 = reinterpret_cast<u32*>(&sh.m.order[1][0]);
    static_assert(sizeof(sh.m.order[1]) + sizeof(sh.m.order[2]) == kLocalMax * sizeof(u32), "one range");
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 e = (u32)local_slot(j);
        sh.m.order[0][arr[j]] = (uint16_t)e;
        sh.m.tag[e] = e < nc ? 0 : kPadTag;
        if constexpr (kOther > 1) wait2[e] = key2[j];
    }
    // The other orders: stable sorts of (key - min, slot) from slot order.
    if constexpr (kOther > 0) {
        u32 pay[kLocalItems];
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) pay[j] = (u32)local_slot(j);
        rec_sort(key, pay, vbits[1], s);
        if constexpr (kOther > 1) {
#pragma unroll
            for (int j = 0; j < kLocalItems; ++j) key[j] = wait2[local_slot(j)];
            __syncthreads();  // dB's keys read before role 1's order overwrites them
        }
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) sh.m.order[1][local_slot(j)] = (uint16_t)pay[j];
        if constexpr (kOther > 1) {
#pragma unroll
            for (int j = 0; j < kLocalItems; ++j) pay[j] = (u32)local_slot(j);
            rec_sort(key, pay, vbits[2], s);
#pragma unroll
            for (int j = 0; j < kLocalItems; ++j) sh.m.order[2][local_slot(j)] = (uint16_t)pay[j];
        }
    }
    __syncthreads();

    const Geometry lg = make_geometry((i64)nc);
    const int rounds = lg.levels - 1;
    // round t splits dimension (l0 + t) mod k, whose role is (t + 1) mod k
    for (int t = 0; t < rounds; ++t) rec_round(sh.m.order[(t + 1) % kK], t, lg, sh.m.tag, s);

    // Level-order output: each point's record (read again, one vector) goes
    // to its node's row in LDS; the nodes of a local level are one
    // contiguous range of global ids ((c << level) + node), written a word
    // per thread.
    u32 node[kLocalItems];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) node[j] = sh.m.tag[sh.m.order[0][local_slot(j)]];
    __syncthreads();  // the rows overlay the tags and orders
    constexpr int kBatch = 4;  // records in flight at once
#pragma unroll
    for (int j0 = 0; j0 < kLocalItems; j0 += kBatch) {
        u32 r[kBatch][4];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            r[j][0] = r[j][1] = r[j][2] = r[j][3] = 0;
            load_record((u32)local_slot(j0 + j), reinterpret_cast<u32(&)[kW]>(r[j]));
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if ((u32)local_slot(j0 + j) < nc) sh.rows[node[j0 + j]] = make_uint4(r[j][0], r[j][1], r[j][2], r[j][3]);
    }
    __syncthreads();
    auto word_of = [&](u32 n, int f) -> u32 {
        const uint4 v = sh.rows[n];
        return f == 0 ? v.x : f == 1 ? v.y : f == 2 ? v.z : v.w;
    };
    for (u32 n = threadIdx.x; n < nc; n += kLocalBlock) {
        const u64 g = (c << level_of(n)) + n;
        if (g < (u64)a.n) a.perm[g] = (int32_t)word_of(n, kK);
    }
    if (a.tree) {
        for (u32 f = threadIdx.x; f < (u32)kK * nc; f += kLocalBlock) {
            const u32 n = f / kK, dim = f - n * kK;
            const u64 g = (c << level_of(n)) + n;
            if (g >= (u64)a.n) continue;
            const u32 key = word_of(n, (int)dim);
            // a zero key (both zeros have it) is read back from the row,
            // which keeps the sign of zero
            const float x = key == 0x80000000u ? a.pts[(u64)word_of(n, kK) * kK + dim]
                                               : __uint_as_float(key_bits(key));
            a.tree[g * kK + dim] = x;
        }
    }
}

// ------------------------------------ subtree stage from staged columns
// The subtree stage when the records do not carry every coordinate (k >
// kCachedDims, or fewer global rounds than k), or when the whole tree is one
// subtree read from the rows (l0 = 0). Each point's index and the keys of
// the dimensions the local rounds split (at most kLocalRounds of them) are
// staged once, by slot (index rank), as columns of the workspace; each
// round then sorts its dimension's column in LDS, as the record stage does
// (value less its minimum, only the bits that differ, a 32-bit word a
// pass), and ranks the points with rec_round. Only the round's own order is
// kept, which leaves 37 KB of LDS a workgroup (its ~120 registers a thread
// allow two workgroups a compute unit either way). The tree rows of the
// output are copied from the points themselves, a level's nodes being one
// contiguous range of rows.
constexpr int kLocalRounds = 12;  // rounds of a kLocalMax-point subtree (13 levels)
static_assert(kLocalMax == 1 << kLocalRounds, "levels of the largest subtree");

struct ColScratch {
    u32 exch[1][kLocalMax];               // record exchange; the rounds' segment counters
    uint16_t count[kLocalWaves][kRadix];  // per-wave digit counters of a pass
    u32 start[kRadix];
    u32 wave[kLocalWaves];
    u32 red[2][kLocalWaves];              // per-wave minimum and maximum
    uint16_t dummy[64];
};

struct ColShared {
    uint16_t tag[kLocalMax];    // local tag of each slot
    uint16_t order[kLocalMax];  // the round's order: slots by (coordinate, index); during its
                                // sort, the payload exchange of the wide passes
    ColScratch s;
};

__global__ __launch_bounds__(kLocalBlock, 4) void k_subtree_cols(SubtreeArgs a) {
    __shared__ ColShared sh;
    ColScratch& s = sh.s;

    const u64 c = full_nodes(a.l0) + blockIdx.x;  // subtree root (global node id)
    const u32 nc = (u32)subtree_size(a.geo, c);
    if (nc == 0) return;
    u64 first = 0;  // live position of the subtree's first point in round l0-1's order
    if (a.l0 > 0) {
        const u64 parent = (c - 1) / 2;
        const u64 seg = live_begin(a.geo, parent - full_nodes(a.l0 - 1), a.l0 - 1);
        first = c == 2 * parent + 1 ? seg : seg + subtree_size(a.geo, 2 * parent + 1) + 1;
    }
    auto rec = [&](u32 q, int f) -> u32 { return a.recs[rec_word_index(a.words, a.plane, first + q, f)]; };
    const int kr = a.recs && !a.index_only ? a.words - 1 : 0;  // coordinates the records carry
    // the arrival order is (coordinate d_a, index)
    const int d_a = a.recs && !a.index_only ? (a.l0 - 1) % a.k : -1;
    const Geometry lg = make_geometry((i64)nc);
    const int rounds = lg.levels - 1;
    const int used = rounds < a.k ? rounds : a.k;  // dimensions (l0 + t) mod k, t < used, differ
    const int d0 = a.l0 % a.k;
    u32* col_idx = a.stage + first;
    // column of the u-th dimension the rounds split, (d0 + u) mod k
    auto column = [&](int u) { return a.stage + (u64)(u + 1) * (u64)a.n + first; };

    // Slot = index rank: sort (index - min, arrival position). arr[j] is the
    // arrival position of slot local_slot(j); the padding positions (q >= nc)
    // sort last, in order, so that slot e >= nc holds arrival position e.
    // Index-only records arrive by index: slot = arrival.
    u32 arr[kLocalItems];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) arr[j] = (u32)local_slot(j);
    if (a.recs && !a.index_only) {
        u32 v[kLocalItems], mn[1] = {~0u}, mx[1] = {0u};
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const u32 q = (u32)local_slot(j);
            v[j] = q < nc ? rec(q, a.words - 1) : 0u;
            mn[0] = q < nc && v[j] < mn[0] ? v[j] : mn[0];
            mx[0] = q < nc && v[j] > mx[0] ? v[j] : mx[0];
        }
        rec_min_max<1>(mn, mx, s);
        const int vbits = value_bits(mx[0] - mn[0]);
        const u32 pad = vbits == 32 ? ~0u : (1u << vbits) - 1;
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) v[j] = (u32)local_slot(j) < nc ? v[j] - mn[0] : pad;
        rec_sort(v, arr, vbits, s, sh.order);
    }

    // Stage by slot. The record words -- the index, and the coordinates
    // below kr -- are read coalesced by arrival position and put in slot
    // order through LDS; for d_a the column holds the arrival position
    // itself, from which its order is known without a sort. The other
    // coordinates the rounds split are the run [d0, d0 + nr) of each row
    // (the used dimensions from d0 on, up to kr's wrap), gathered two points
    // at a time with a point's loads issued together, so that a row is
    // fetched once.
    uint16_t* slot_of_arr = sh.order;  // free until the first round
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) slot_of_arr[arr[j]] = (uint16_t)local_slot(j);
    __syncthreads();  // (also orders the sort's last exchange reads before its reuse)
    auto stage_word = [&](int f, u32* dst, u32 (&got)[kLocalItems]) {
        u32 val[kLocalItems];
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const u32 q = (u32)local_slot(j);
            val[j] = q < nc ? rec(q, f) : 0u;
        }
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) s.exch[0][slot_of_arr[local_slot(j)]] = val[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const u32 e = (u32)local_slot(j);
            got[j] = s.exch[0][e];
            if (e < nc) dst[e] = got[j];
        }
        __syncthreads();
    };
    u32 idx[kLocalItems];  // index of the point in slot local_slot(j)
    if (a.recs) {
        stage_word(a.words - 1, col_idx, idx);
    } else {
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const u32 e = (u32)local_slot(j);
            idx[j] = e;
            if (e < nc) col_idx[e] = e;
        }
    }
    // kr = min(k, l0) and d0 = l0 mod k: below k global rounds kr = d0, and
    // the used dimensions from d0 to k-1 come from the rows, the wrapped
    // ones (below kr) from the records; records of the index alone: every
    // used dimension from the rows, wrapping past k-1 to 0
    const int nr = kr == a.k ? 0 : (kr == 0 ? used : (used < a.k - d0 ? used : a.k - d0));
    for (int u = nr, d = (d0 + nr) % a.k; u < used; ++u, d = d + 1 == a.k ? 0 : d + 1) {
        if (d == d_a) {
#pragma unroll
            for (int j = 0; j < kLocalItems; ++j)
                if ((u32)local_slot(j) < nc) column(u)[local_slot(j)] = arr[j];
        } else {
            u32 got[kLocalItems];
            stage_word(d, column(u), got);
        }
    }
    if (nr > 0) {
#pragma unroll
        for (int j0 = 0; j0 < kLocalItems; j0 += 2) {
            u32 key[2][kLocalRounds];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bool ok = (u32)local_slot(j0 + h) < nc;
                const float* row = a.pts + (u64)idx[j0 + h] * (u64)a.k;
#pragma unroll
                for (int i = 0; i < kLocalRounds; ++i) {
                    const int dd = d0 + i < a.k ? d0 + i : d0 + i - a.k;
                    key[h][i] = ok && i < nr ? float_key(__float_as_uint(row[dd])) : 0u;
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32 e = (u32)local_slot(j0 + h);
                if (e >= nc) continue;
                u32* dst = column(0) + e;
#pragma unroll
                for (int i = 0; i < kLocalRounds; ++i)
                    if (i < nr) dst[(u64)i * (u64)a.n] = key[h][i];
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) sh.tag[local_slot(j)] = (u32)local_slot(j) < nc ? 0 : kPadTag;
    __syncthreads();  // the columns written before a round reads them; the tags set

    int d = d0, u = 0;  // round t splits dimension d, staged in column u = t mod k
    for (int t = 0; t < rounds; ++t) {
        const u32* col = column(u);
        if (d == d_a) {
            // order[q] = slot of arrival position q
#pragma unroll
            for (int j = 0; j < kLocalItems; ++j) {
                const u32 e = (u32)local_slot(j);
                sh.order[e < nc ? col[e] : e] = (uint16_t)e;
            }
        } else {
            u32 v[kLocalItems], pay[kLocalItems], mn[1] = {~0u}, mx[1] = {0u};
#pragma unroll
            for (int j = 0; j < kLocalItems; ++j) {
                const u32 e = (u32)local_slot(j);
                v[j] = e < nc ? col[e] : 0u;
                mn[0] = e < nc && v[j] < mn[0] ? v[j] : mn[0];
                mx[0] = e < nc && v[j] > mx[0] ? v[j] : mx[0];
                pay[j] = e;
            }
            rec_min_max<1>(mn, mx, s);
            const int vbits = value_bits(mx[0] - mn[0]);
            const u32 pad = vbits == 32 ? ~0u : (1u << vbits) - 1;
#pragma unroll
            for (int j = 0; j < kLocalItems; ++j) v[j] = (u32)local_slot(j) < nc ? v[j] - mn[0] : pad;
            // (the sort's last pass reads only the word exchange: order is free)
            rec_sort(v, pay, vbits, s, sh.order);
#pragma unroll
            for (int j = 0; j < kLocalItems; ++j) sh.order[local_slot(j)] = (uint16_t)pay[j];
        }
        __syncthreads();
        // 16-bit counters fill the exchange buffer at 1024 segments; past
        // that a segment holds at most 3 points
        if ((size_t)kLocalWaves * sizeof(uint16_t) << t <= sizeof(s.exch))
            rec_round<uint16_t>(sh.order, t, lg, sh.tag, s);
        else
            rec_round<uint8_t>(sh.order, t, lg, sh.tag, s);
        d = d + 1 == a.k ? 0 : d + 1;
        u = u + 1 == a.k ? 0 : u + 1;
    }

    // Output: the index of each local node (by its final tag), then perm and
    // the tree rows, a level's nodes being the contiguous global range
    // (c << level) + node.
    u32* idx_of = s.exch[0];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 e = (u32)local_slot(j);
        if (e < nc) idx_of[sh.tag[e]] = col_idx[e];
    }
    __syncthreads();
    for (u32 n = threadIdx.x; n < nc; n += kLocalBlock) {
        const u64 g = (c << level_of(n)) + n;
        if (g < (u64)a.n) a.perm[g] = (int32_t)idx_of[n];
    }
    if (!a.tree) return;
    // word f = n k + dim of the subtree's rows, node n = f / k stepped along
    const u32 k = (u32)a.k, total = k * nc;
    const u32 step_n = kLocalBlock / k, step_d = kLocalBlock % k;
    u32 n = threadIdx.x / k, dim = threadIdx.x % k;
    for (u32 f = threadIdx.x; f < total; f += kLocalBlock) {
        const u64 g = (c << level_of(n)) + n;
        if (g < (u64)a.n) a.tree[g * k + dim] = a.pts[(u64)idx_of[n] * k + dim];
        n += step_n;
        dim += step_d;
        if (dim >= k) {
            dim -= k;
            ++n;
        }
    }
}

// ------------------------------- split-widest subtrees finished in LDS
// The subtree stage for split-widest trees (k <= kCachedDims): the order of
// every dimension is kept, and a level's nodes are ranked in one sub-round
// per dimension, over that dimension's order and only for the segments
// whose node splits it. After a level, the thread holding each node's pivot
// derives the children's domains and split dimensions (child_domain, as on
// the global levels). The subtree's records are A_0's on level l0 (in
// (coordinate 0, index) order), or the rows themselves when the whole tree
// is one subtree.
struct WidestSubtreeArgs {
    const float* pts;
    i64 n;
    int k;
    int l0;                  // level of the subtree roots
    Geometry geo;
    const u32* recs;         // l0 > 0: A_0 on level l0 (k keys, then the index); nullptr: rows
    float* boxes;            // N x 2k domains: the roots' are there; the stage writes its nodes'
    const uint16_t* dimtab;  // the roots' split dimensions
    int32_t* perm;
    float* tree;
    int32_t* dims_out;
};

// The live points of level t of a split-widest subtree as one list: for each
// dimension d that some level-t node splits, in turn, the slots of the
// points whose node splits d, in the order of d. Each node's points are then
// in its own dimension's order, and one round over the list ranks them all.
// A first pass looks up each slot's node dimension once (0xff: no point of
// level t), in exch[0], so that each dimension's pass makes one gather an
// item. Returns the list's length (uniform).
__device__ __forceinline__ u32 rec_live_list(RecShared& sh, const uint8_t* nodedim, u32 used, int t, int dims,
                                             uint16_t* list) {
    RecScratch& s = sh.m.s;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const u32 fl = (1u << t) - 1, segs = 1u << t;
    uint8_t* sdim = reinterpret_cast<uint8_t*>(&s.exch[0][0]);
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 e = (u32)local_slot(j);
        const u32 st = sh.m.tag[e];  // (padding: kPadTag, on no level)
        const bool on = st - fl < segs;
        const uint8_t nd = nodedim[on ? st : 0u];
        sdim[e] = on ? nd : (uint8_t)0xff;
    }
    __syncthreads();
    u32 base = 0;
    for (int d = 0; d < dims; ++d) {
        if (!((used >> d) & 1u)) continue;
        u32 e[kLocalItems];
        u64 keep[kLocalItems];
        u32 wave_total = 0;
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) e[j] = sh.m.order[d][local_slot(j)];
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            keep[j] = __ballot(sdim[e[j]] == (uint8_t)d);
            wave_total += (u32)__popcll(keep[j]);
        }
        if (lane == 0) s.wave[w] = wave_total;
        __syncthreads();
        u32 at = base, total = 0;
#pragma unroll
        for (int v = 0; v < kLocalWaves; ++v) {
            const u32 c = s.wave[v];
            at += v < w ? c : 0u;
            total += c;
        }
        // (items not kept write to a dummy: no branch an item)
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const bool kept = (keep[j] >> lane) & 1u;
            uint16_t* to = kept ? &list[at + lanes_below((u32)keep[j], (u32)(keep[j] >> 32))] : &s.dummy[lane];
            *to = (uint16_t)e[j];
            at += (u32)__popcll(keep[j]);
        }
        base += total;
        __syncthreads();  // s.wave read before the next dimension writes it
    }
    return base;
}

// Round t over such a list of n_live slots, as rec_round with every listed
// point live. Per-wave segment counters of type Count (16-bit, or 8-bit on
// levels whose segments hold at most 255 points) in exch[0].
// kT >= 0: the round index as a compile-time constant (t_rt unused), so that
// the t-bit ballot match unrolls.
template <int kT, typename Count>
__device__ __forceinline__ void rec_round_list_at(const uint16_t* list, u32 n_live, int t_rt, const Geometry& lg,
                                                  RecShared& sh) {
    const int t = kT >= 0 ? kT : t_rt;
    RecScratch& s = sh.m.s;
    // (thread-derived offsets recomputed a call, not held across the level loop)
    const int tid = (int)opaque(threadIdx.x), lane = tid & 63, w = tid >> 6;
    const u32 fl = (1u << t) - 1, segs = 1u << t;
    constexpr u32 kPer = 4 / sizeof(Count);  // counters a word
    Count* cnt = reinterpret_cast<Count*>(&s.exch[0][0]);  // [kLocalWaves][segs]
    u32* cnt_words = &s.exch[0][0];
    const u32 words = (kLocalWaves * segs + kPer - 1) / kPer;
    for (u32 i = tid; i < words; i += kLocalBlock) cnt_words[i] = 0;
    __syncthreads();
    u32 e[kLocalItems], st[kLocalItems], rank[kLocalItems];
    bool in[kLocalItems];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        in[j] = (u32)local_slot(j) < n_live;
        e[j] = in[j] ? list[local_slot(j)] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) st[j] = in[j] ? sh.m.tag[e[j]] : fl;
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 b = st[j] - fl;
        const u64 lv = __ballot(in[j]);
        u32 p_lo, p_hi;
        peer_mask(b, t, (u32)lv, (u32)(lv >> 32), p_lo, p_hi);
        const u32 before = lanes_below(p_lo, p_hi);
        Count* cp = in[j] ? &cnt[w * segs + b] : reinterpret_cast<Count*>(&s.dummy[lane]);
        const u32 seen = *cp;
        rank[j] = seen + before;
        *cp = (Count)(seen + __popc(p_lo) + __popc(p_hi));
    }
    __syncthreads();
    // prefix over the waves, kPer counters a word (a segment's total fits
    // one counter, so the lanes of a word never carry into each other)
    if (segs >= kPer) {
        const u32 row = segs / kPer;
        for (u32 i = tid; i < row; i += kLocalBlock) {
            u32 run = 0;
#pragma unroll
            for (int v = 0; v < kLocalWaves; ++v) {
                const u32 c = cnt_words[v * row + i];
                cnt_words[v * row + i] = run;
                run += c;
            }
        }
    } else if (tid < (int)segs) {
        u32 run = 0;
#pragma unroll
        for (int v = 0; v < kLocalWaves; ++v) {
            const u32 c = cnt[v * segs + tid];
            cnt[v * segs + tid] = (Count)run;
            run += c;
        }
    }
    __syncthreads();
    const u32 dd = (u32)(lg.levels - 2 - t), u = 1u << dd, last = (u32)lg.last;
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) rank[j] += in[j] ? (u32)cnt[w * segs + (st[j] - fl)] : 0u;
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        if (!in[j]) continue;
        const u32 b = st[j] - fl;
        const u32 in_seg = rank[j];
        const u32 under = (2 * b) << dd;
        const u32 left = (u - 1) + (last > under ? (last - under < u ? last - under : u) : 0u);
        const u32 next = in_seg < left ? 2 * st[j] + 1 : (in_seg > left ? 2 * st[j] + 2 : st[j]);
        sh.m.tag[e[j]] = (uint16_t)next;
    }
    __syncthreads();
}

template <typename Count>
__device__ __forceinline__ void rec_round_list(const uint16_t* list, u32 n_live, int t, const Geometry& lg,
                                               RecShared& sh) {
    switch (t) {  // every round of a kLocalMax-point subtree: t <= kLocalRounds - 1
#define KDT_LIST_ROUND_CASE(T) \
    case T: rec_round_list_at<T, Count>(list, n_live, t, lg, sh); break;
        KDT_LIST_ROUND_CASE(0) KDT_LIST_ROUND_CASE(1) KDT_LIST_ROUND_CASE(2) KDT_LIST_ROUND_CASE(3)
        KDT_LIST_ROUND_CASE(4) KDT_LIST_ROUND_CASE(5) KDT_LIST_ROUND_CASE(6) KDT_LIST_ROUND_CASE(7)
        KDT_LIST_ROUND_CASE(8) KDT_LIST_ROUND_CASE(9) KDT_LIST_ROUND_CASE(10) KDT_LIST_ROUND_CASE(11)
#undef KDT_LIST_ROUND_CASE
        default: rec_round_list_at<-1, Count>(list, n_live, t, lg, sh); break;
    }
}

struct WidestRecShared {
    RecShared r;
    uint8_t nodedim[kLocalMax];  // split dimension of each local node
    u32 dim_mask[2];             // dimensions split on a level (by level parity)
};

template <int kK>
__global__ __launch_bounds__(kLocalBlock, 4) void k_subtree_widest(WidestSubtreeArgs a) {
    static_assert(kK >= 1 && kK <= kCachedDims, "every coordinate in the record");
    constexpr int kW = kK + 1;  // record words: the keys, then the index
    __shared__ WidestRecShared wsh;
    RecShared& sh = wsh.r;
    RecScratch& s = sh.m.s;

    const u64 c = full_nodes(a.l0) + blockIdx.x;  // subtree root (global node id)
    const u32 nc = (u32)subtree_size(a.geo, c);
    if (nc == 0) return;
    // Records of A_0 on level l0 arrive by (coordinate 0, index); the rows
    // (the whole tree as one subtree) arrive by index.
    const bool rows = a.recs == nullptr;
    const u64 first = rows ? 0 : live_begin(a.geo, c - full_nodes(a.l0), a.l0);
    const u32* recs = rows ? nullptr : a.recs + first * kW;
    auto load_record = [&](u32 q, u32 (&r)[4]) {
        const u32 qq = q < nc ? q : nc - 1;
        if (rows) {
#pragma unroll
            for (int f = 0; f < kK; ++f) r[f] = float_key(__float_as_uint(a.pts[(u64)qq * kK + f]));
            r[kK] = qq;
        } else if constexpr (kW == 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(recs + (u64)qq * kW);
            r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
        } else if constexpr (kW == 2) {
            const uint2 v = *reinterpret_cast<const uint2*>(recs + (u64)qq * kW);
            r[0] = v.x; r[1] = v.y;
        } else {
#pragma unroll
            for (int f = 0; f < kW; ++f) r[f] = recs[(u64)qq * kW + f];
        }
    };
    auto pick = [](const u32 (&r)[4], int f) {
        return f == 0 ? r[0] : f == 1 ? r[1] : f == 2 ? r[2] : r[3];
    };
    // Keys that wait by arrival position while the slots are sorted.
    u32* stash = reinterpret_cast<u32*>(&sh.m.tag[0]);
    static_assert(sizeof(sh.m.tag) + sizeof(sh.m.order) >= 2 * kLocalMax * sizeof(u32), "stash");

    // arr[j]: arrival position of the point in slot local_slot(j) (slot =
    // index rank); kept for reading a pivot's coordinate back.
    u32 arr[kLocalItems];
    if (rows) {
        // Slot = arrival: each dimension's order is a stable sort of
        // (key - min, slot), its keys read from the rows by slot.
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const u32 e = (u32)local_slot(j);
            arr[j] = e;
            sh.m.tag[e] = e < nc ? 0 : kPadTag;
        }
        for (int d = 0; d < kK; ++d) {
            u32 key[kLocalItems], pay[kLocalItems];
            u32 mn[1] = {~0u}, mx[1] = {0u};
#pragma unroll
            for (int j = 0; j < kLocalItems; ++j) {
                const u32 e = (u32)local_slot(j);
                key[j] = float_key(__float_as_uint(a.pts[(u64)(e < nc ? e : nc - 1) * kK + d]));
                if (e < nc) {
                    mn[0] = key[j] < mn[0] ? key[j] : mn[0];
                    mx[0] = key[j] > mx[0] ? key[j] : mx[0];
                }
            }
            rec_min_max<1>(mn, mx, s);
            const int vbits = value_bits(mx[0] - mn[0]);
            const u32 pad = vbits == 32 ? ~0u : (1u << vbits) - 1;
#pragma unroll
            for (int j = 0; j < kLocalItems; ++j) {
                const u32 e = (u32)local_slot(j);
                key[j] = e < nc ? key[j] - mn[0] : pad;
                pay[j] = e;
            }
            rec_sort(key, pay, vbits, s);
#pragma unroll
            for (int j = 0; j < kLocalItems; ++j) sh.m.order[d][local_slot(j)] = (uint16_t)pay[j];
        }
    } else {
        // As the round-robin stage with dimension 0 arrived: one vector load
        // per record; dimensions 1 and 2 wait in the stash.
        constexpr int kOther = kK - 1;
        u32 idx[kLocalItems];
        u32 mn[1 + kOther], mx[1 + kOther];
#pragma unroll
        for (int i = 0; i <= kOther; ++i) {
            mn[i] = ~0u;
            mx[i] = 0;
        }
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const u32 q = (u32)local_slot(j);
            u32 r[4] = {0, 0, 0, 0};
            load_record(q, r);
            const bool ok = q < nc;
            idx[j] = r[kK];
            mn[0] = ok && idx[j] < mn[0] ? idx[j] : mn[0];
            mx[0] = ok && idx[j] > mx[0] ? idx[j] : mx[0];
#pragma unroll
            for (int u = 0; u < kOther; ++u) {
                const u32 key = pick(r, 1 + u);
                stash[u * kLocalMax + q] = key;
                mn[1 + u] = ok && key < mn[1 + u] ? key : mn[1 + u];
                mx[1 + u] = ok && key > mx[1 + u] ? key : mx[1 + u];
            }
        }
        rec_min_max<1 + kOther>(mn, mx, s);
        int vbits[1 + kOther];
        u32 pad[1 + kOther];
#pragma unroll
        for (int i = 0; i <= kOther; ++i) {
            vbits[i] = value_bits(mx[i] - mn[i]);
            pad[i] = vbits[i] == 32 ? ~0u : (1u << vbits[i]) - 1;
        }
        {
            u32 v[kLocalItems];
#pragma unroll
            for (int j = 0; j < kLocalItems; ++j) {
                const u32 q = (u32)local_slot(j);
                v[j] = q < nc ? idx[j] - mn[0] : pad[0];
                arr[j] = q;
            }
            rec_sort(v, arr, vbits[0], s);
        }
        u32 key[kLocalItems], key2[kLocalItems];
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const bool ok = (u32)local_slot(j) < nc;
            if constexpr (kOther > 0) key[j] = ok ? stash[arr[j]] - mn[1] : pad[1];
            if constexpr (kOther > 1) key2[j] = ok ? stash[kLocalMax + arr[j]] - mn[2] : pad[2];
        }
        __syncthreads();  // stash read before the tags and orders overwrite it
        u32* wait2 = reinterpret_cast<u32*>(&sh.m.order[1][0]);
        static_assert(sizeof(sh.m.order[1]) + sizeof(sh.m.order[2]) == kLocalMax * sizeof(u32), "one range");
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const u32 e = (u32)local_slot(j);
            sh.m.order[0][arr[j]] = (uint16_t)e;
            sh.m.tag[e] = e < nc ? 0 : kPadTag;
            if constexpr (kOther > 1) wait2[e] = key2[j];
        }
        if constexpr (kOther > 0) {
            u32 pay[kLocalItems];
#pragma unroll
            for (int j = 0; j < kLocalItems; ++j) pay[j] = (u32)local_slot(j);
            rec_sort(key, pay, vbits[1], s);
            if constexpr (kOther > 1) {
#pragma unroll
                for (int j = 0; j < kLocalItems; ++j) key[j] = wait2[local_slot(j)];
                __syncthreads();  // dimension 2's keys read before order 1 overwrites them
            }
#pragma unroll
            for (int j = 0; j < kLocalItems; ++j) sh.m.order[1][local_slot(j)] = (uint16_t)pay[j];
            if constexpr (kOther > 1) {
#pragma unroll
                for (int j = 0; j < kLocalItems; ++j) pay[j] = (u32)local_slot(j);
                rec_sort(key, pay, vbits[2], s);
#pragma unroll
                for (int j = 0; j < kLocalItems; ++j) sh.m.order[2][local_slot(j)] = (uint16_t)pay[j];
            }
        }
    }
    // From here on arr[j] is the byte offset of that point's record (or
    // row) from `src`: a 32-bit offset to a uniform base, not a pointer per
    // slot.
    const char* src = rows ? reinterpret_cast<const char*>(a.pts) : reinterpret_cast<const char*>(recs);
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) arr[j] *= (rows ? kK : kW) * 4u;
    if (threadIdx.x == 0) {
        wsh.nodedim[0] = (uint8_t)a.dimtab[c];
        wsh.dim_mask[0] = 1u << a.dimtab[c];
    }
    __syncthreads();

    const Geometry lg = make_geometry((i64)nc);
    const int rounds = lg.levels - 1;
    for (int t = 0; t < rounds; ++t) {
        const u32 fl = (u32)full_nodes(t), fl1 = (u32)full_nodes(t + 1);
        const u32 used = wsh.dim_mask[t & 1];  // dimensions this level's nodes split
        if (threadIdx.x == 0) wsh.dim_mask[(t + 1) & 1] = 0;  // read a level ago; the rounds' barriers follow
        if (__popc(used) == 1) {  // one dimension: its order is the list
            rec_round(sh.m.order[__ffs(used) - 1], t, lg, sh.m.tag, s, wsh.nodedim, (u32)(__ffs(used) - 1));
        } else {
            // the list in exch[1], the counters in exch[0] (16 KB: 16-bit
            // up to 1024 segments; 8-bit where a segment holds at most 255
            // points, which is every level with more segments)
            uint16_t* list = reinterpret_cast<uint16_t*>(&s.exch[1][0]);
            const u32 n_live = rec_live_list(sh, wsh.nodedim, used, t, kK, list);
            if (lg.levels - t <= 8) rec_round_list<uint8_t>(list, n_live, t, lg, sh);
            else rec_round_list<uint16_t>(list, n_live, t, lg, sh);
        }
        // Level t's pivots carry their node's tag now. Each pivot's thread
        // leaves its coordinate in its node's dimension in LDS (the round's
        // counters are dead), then one thread a node bounds the node's domain
        // at that plane for both children and picks their dimensions.
        const u32 nodes = fl1 - fl;
        float* plane_of = reinterpret_cast<float*>(&s.exch[0][0]);  // [nodes]
        const u64 level_first = ((c + 1) << t) - 1;  // global id of local node fl
        float lo[kK], hi[kK];
        auto load_domain = [&](u32 i) {
            const float* from = a.boxes + (level_first + i) * 2 * (u64)kK;
#pragma unroll
            for (int d = 0; d < kK; ++d) {
                lo[d] = from[d];
                hi[d] = from[kK + d];
            }
        };
        // (the first node's domain is in flight during the pivots' pass)
        if (threadIdx.x < nodes && 2 * (fl + threadIdx.x) + 1 < nc) load_domain(threadIdx.x);
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const u32 e = (u32)local_slot(j);
            const u32 sn = sh.m.tag[e];  // (padding: kPadTag, above every level)
            if (sn - fl >= nodes) continue;
            // the pivot's coordinate (a zero's sign: the extents agree)
            u32 pkey = *reinterpret_cast<const u32*>(src + (arr[j] + 4u * (u32)wsh.nodedim[sn]));
            if (rows) pkey = float_key(pkey);
            plane_of[sn - fl] = __uint_as_float(key_bits(pkey));
        }
        __syncthreads();
        u32 split_bits = 0;  // dimensions this thread's children split
        for (u32 i = threadIdx.x; i < nodes; i += kLocalBlock) {
            const u32 sn = fl + i;
            if (2 * sn + 1 >= nc) break;  // a leaf, as is every later node of the level
            if (i != threadIdx.x) load_domain(i);
            const int ds = wsh.nodedim[sn];
            const float plane = plane_of[i];
            for (u32 ch = 2 * sn + 1; ch <= 2 * sn + 2 && ch < nc; ++ch) {
                const u64 g = (((c + 1) << (t + 1)) - 1) + (ch - fl1);
                const bool left = ch == 2 * sn + 1;
                float clo[kK], chi[kK];
                int best = 0;
                float best_extent = 0.0f;
#pragma unroll
                for (int d = 0; d < kK; ++d) {
                    clo[d] = lo[d];
                    chi[d] = hi[d];
                    if (d == ds) {
                        if (left) chi[d] = plane;
                        else clo[d] = plane;
                    }
                    const float extent = chi[d] - clo[d];
                    if (d == 0 || extent > best_extent) {
                        best = d;
                        best_extent = extent;
                    }
                }
                if (t + 1 < rounds) {  // a parent in the next round: keep its domain
                    float* box = a.boxes + g * 2 * (u64)kK;
#pragma unroll
                    for (int d = 0; d < kK; ++d) {
                        box[d] = clo[d];
                        box[kK + d] = chi[d];
                    }
                }
                wsh.nodedim[ch] = (uint8_t)best;
                split_bits |= 1u << best;
                if (a.dims_out) a.dims_out[g] = best;
            }
        }
        // one LDS atomic a wave
        u32 wave_bits = 0;
#pragma unroll
        for (int d = 0; d < kK; ++d) wave_bits |= __ballot((split_bits >> d) & 1u) != 0 ? 1u << d : 0u;
        if ((threadIdx.x & 63) == 0 && wave_bits) atomicOr(&wsh.dim_mask[(t + 1) & 1], wave_bits);
        __syncthreads();
    }

    // Level-order output as in the round-robin stage: each point's record
    // (read again) goes to its node's row in LDS, then out by node.
    u32 node[kLocalItems];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 q = (u32)local_slot(j);
        node[j] = sh.m.tag[rows ? q : sh.m.order[0][q]];
    }
    __syncthreads();  // the rows overlay the tags and orders
    constexpr int kBatch = 4;  // records in flight at once
#pragma unroll
    for (int j0 = 0; j0 < kLocalItems; j0 += kBatch) {
        u32 r[kBatch][4];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            r[j][0] = r[j][1] = r[j][2] = r[j][3] = 0;
            load_record((u32)local_slot(j0 + j), r[j]);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if ((u32)local_slot(j0 + j) < nc) sh.rows[node[j0 + j]] = make_uint4(r[j][0], r[j][1], r[j][2], r[j][3]);
    }
    __syncthreads();
    auto word_of = [&](u32 n, int f) -> u32 {
        const uint4 v = sh.rows[n];
        return f == 0 ? v.x : f == 1 ? v.y : f == 2 ? v.z : v.w;
    };
    for (u32 n = threadIdx.x; n < nc; n += kLocalBlock) {
        const u64 g = ((c + 1) << level_of(n)) - 1 + (n - full_nodes(level_of(n)));
        a.perm[g] = (int32_t)word_of(n, kK);
    }
    if (a.tree) {
        for (u32 f = threadIdx.x; f < (u32)kK * nc; f += kLocalBlock) {
            const u32 n = f / kK, dim = f - n * kK;
            const u64 g = ((c + 1) << level_of(n)) - 1 + (n - full_nodes(level_of(n)));
            const u32 key = word_of(n, (int)dim);
            // a zero key (both zeros have it) is read back from the row,
            // which keeps the sign of zero
            a.tree[g * kK + dim] = key == 0x80000000u ? a.pts[(u64)word_of(n, kK) * kK + dim]
                                                      : __uint_as_float(key_bits(key));
        }
    }
}

// ------------------------- split-widest subtrees with more than 3 dimensions
// The subtree stage of split-widest trees for k > kCachedDims, where no
// order of every dimension fits LDS. A round ranks each node's points by its
// own split dimension only within the node's segment, so one sort per level
// of every live point by the key of its node's dimension (keys of different
// dimensions interleave, but never within a segment) gives every segment its
// order: each level is one sort and one round, as in the columns stage. The
// keys are read from the subtree's records of A_0 (planar: coordinate d in
// plane d) at each point's arrival position, kept in LDS by slot; the node
// dimensions (16-bit: k up to 65535) are in LDS too, and after each round
// the thread holding a new pivot derives both children's domains and
// dimensions with child_domain, as the global levels do. The whole tree as
// one subtree (l0 = 0) reads the rows instead.
struct WidestColShared {
    ColShared c;
    uint16_t nodedim[kLocalMax];  // split dimension of each local node
    uint16_t arr[kLocalMax];      // arrival position of each slot
};

__global__ __launch_bounds__(kLocalBlock, 4) void k_subtree_widest_cols(WidestSubtreeArgs a) {
    __shared__ WidestColShared sh;
    ColScratch& s = sh.c.s;
    const u64 c = full_nodes(a.l0) + blockIdx.x;  // subtree root (global node id)
    const u32 nc = (u32)subtree_size(a.geo, c);
    if (nc == 0) return;
    const bool rows = a.recs == nullptr;
    const u64 first = rows ? 0 : live_begin(a.geo, c - full_nodes(a.l0), a.l0);
    const u32 k = (u32)a.k;
    // key of coordinate d of the point that arrived at position q (its index
    // i: the rows' case)
    auto key = [&](u32 q, u32 d) -> u32 {
        if (rows) return float_key(__float_as_uint(a.pts[(u64)q * k + d]));
        return a.recs[(u64)d * (u64)a.n + first + q];
    };

    // Slot = index rank: sort (index - min, arrival position); the rows
    // arrive by index.
    u32 arr[kLocalItems];
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) arr[j] = (u32)local_slot(j);
    if (!rows) {
        u32 v[kLocalItems], mn[1] = {~0u}, mx[1] = {0u};
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const u32 q = (u32)local_slot(j);
            v[j] = q < nc ? key(q, k) : 0u;  // word k: the index
            mn[0] = q < nc && v[j] < mn[0] ? v[j] : mn[0];
            mx[0] = q < nc && v[j] > mx[0] ? v[j] : mx[0];
        }
        rec_min_max<1>(mn, mx, s);
        const int vbits = value_bits(mx[0] - mn[0]);
        const u32 pad = vbits == 32 ? ~0u : (1u << vbits) - 1;
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) v[j] = (u32)local_slot(j) < nc ? v[j] - mn[0] : pad;
        rec_sort(v, arr, vbits, s, sh.c.order);
    }
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const int e = local_slot(j);
        sh.arr[e] = (uint16_t)arr[j];
        sh.c.tag[e] = (u32)e < nc ? 0 : kPadTag;
    }
    if (threadIdx.x == 0) sh.nodedim[0] = a.dimtab[c];
    __syncthreads();

    const Geometry lg = make_geometry((i64)nc);
    const int rounds = lg.levels - 1;
    for (int t = 0; t < rounds; ++t) {
        const u32 fl = (u32)full_nodes(t), fl1 = (u32)full_nodes(t + 1);
        // slot of item j: slot0 + 64 j (recomputed each level, not held)
        const u32 slot0 = opaque((u32)local_slot(0));
        // every live point's key in its node's dimension (fixed points and
        // padding sort last: they are not ranked)
        u32 v[kLocalItems], pay[kLocalItems], mn[1] = {~0u}, mx[1] = {0u};
        u32 live = 0;  // bit j: slot slot0 + 64 j holds a point of level t
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            const u32 e = (slot0 + 64u * j);
            const u32 st = sh.c.tag[e];
            const bool on = st - fl < fl1 - fl;
            live |= (u32)on << j;
            v[j] = on ? key(sh.arr[e], sh.nodedim[st]) : 0u;
            mn[0] = on && v[j] < mn[0] ? v[j] : mn[0];
            mx[0] = on && v[j] > mx[0] ? v[j] : mx[0];
        }
        rec_min_max<1>(mn, mx, s);
        const int vbits = value_bits(mx[0] - mn[0]);
        const u32 pad = vbits == 32 ? ~0u : (1u << vbits) - 1;
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) {
            v[j] = (live >> j) & 1u ? v[j] - mn[0] : pad;
            pay[j] = (slot0 + 64u * j);
        }
        rec_sort(v, pay, vbits, s, sh.c.order);
#pragma unroll
        for (int j = 0; j < kLocalItems; ++j) sh.c.order[slot0 + 64u * j] = (uint16_t)pay[j];
        __syncthreads();
        if ((size_t)kLocalWaves * sizeof(uint16_t) << t <= sizeof(s.exch))
            rec_round<uint16_t>(sh.c.order, t, lg, sh.c.tag, s);
        else
            rec_round<uint8_t>(sh.c.order, t, lg, sh.c.tag, s);
        // Level t's pivots carry their node's tag now: each one's thread
        // leaves its coordinate in its node's dimension in LDS (the round's
        // counters are dead), then one thread a node derives both children's
        // domains and dimensions.
        const u32 nodes = fl1 - fl;
        float* plane_of = reinterpret_cast<float*>(&s.exch[0][0]);  // [nodes]
#pragma unroll 1
        for (int j = 0; j < kLocalItems; ++j) {
            const u32 e = (slot0 + 64u * j);
            const u32 sn = sh.c.tag[e];  // (padding: kPadTag, above every level)
            if (sn - fl >= nodes) continue;
            // (a zero's sign: the extents agree)
            plane_of[sn - fl] = __uint_as_float(key_bits(key(sh.arr[e], sh.nodedim[sn])));
        }
        __syncthreads();
        for (u32 i = threadIdx.x; i < nodes; i += kLocalBlock) {
            const u32 sn = fl + i;
            if (2 * sn + 1 >= nc) break;  // a leaf, as is every later node of the level
            const u32 ds = sh.nodedim[sn];
            const float* from = a.boxes + ((((c + 1) << t) - 1) + i) * 2 * (u64)k;
            for (u32 ch = 2 * sn + 1; ch <= 2 * sn + 2 && ch < nc; ++ch) {
                const u64 g = (((c + 1) << (t + 1)) - 1) + (ch - fl1);
                const int best =
                    child_domain(from, (int)ds, plane_of[i], ch == 2 * sn + 1, (int)k, a.boxes + g * 2 * (u64)k);
                sh.nodedim[ch] = (uint16_t)best;
                if (a.dims_out) a.dims_out[g] = best;
            }
        }
        __syncthreads();
    }

    // Output as in the columns stage: each node's index (by its final tag),
    // then perm and the tree rows, a level's nodes being the contiguous
    // global range (c << level) + node.
    u32* idx_of = s.exch[0];
    const u32 slot0 = opaque((u32)local_slot(0));
#pragma unroll
    for (int j = 0; j < kLocalItems; ++j) {
        const u32 e = slot0 + 64u * j;
        if (e < nc) idx_of[sh.c.tag[e]] = rows ? sh.arr[e] : key(sh.arr[e], k);
    }
    __syncthreads();
    for (u32 n = threadIdx.x; n < nc; n += kLocalBlock) {
        const u64 g = (c << level_of(n)) + n;
        if (g < (u64)a.n) a.perm[g] = (int32_t)idx_of[n];
    }
    if (!a.tree) return;
    const u32 total = k * nc;
    const u32 step_n = kLocalBlock / k, step_d = kLocalBlock % k;
    u32 n = threadIdx.x / k, dim = threadIdx.x % k;
    for (u32 f = threadIdx.x; f < total; f += kLocalBlock) {
        const u64 g = (c << level_of(n)) + n;
        if (g < (u64)a.n) a.tree[g * k + dim] = a.pts[(u64)idx_of[n] * k + dim];
        n += step_n;
        dim += step_d;
        if (dim >= k) {
            dim -= k;
            ++n;
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


// ------------------------------------------------------------ host driver

inline size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
    int rounds;          // global rounds: levels fixed before the subtree stage
    int kr;              // coordinates a record carries: dimensions 0 .. kr-1
    int words;           // record width, kr + 1
    int nbuf;            // record arrays
    i64 tiles;           // of a pass over all n points
    size_t tmp0, tmp1, digits, digits0, recs, piv, totals, slots, chunk_slots, stage, total;
    size_t tags;         // rounds by per-point tags (tag_rounds): a tag of each point
    size_t planar0;      // records wider than kWholeWords: all of them in index order, planar
};

// Whether the subtree stage after `rounds` global rounds reads records that
// carry every coordinate (k_subtree_recs) rather than staging columns.
inline bool stage_from_records(int k, int rounds) { return rounds > 0 && k <= rounds && k <= kCachedDims; }

// Whether a build's global rounds run by per-point tags (run_global_tags):
// at least four of them (the planar copy of the rounds' keys exists), k > 3,
// and either every round splits a new dimension (k >= rounds) or k is at
// least kTagDims. Per-dimension arrays cost a pass over each of them per
// round, tags a fixed number of 16-byte passes; normal points, arrays
// against tags: 4M points k = 5 2.53 / 2.90 ms, k = 6 3.07 / 2.98, k = 8
// 4.46 / 3.13; 16M points k = 5 11.28 / 11.48, k = 8 19.92 / 11.99.
constexpr int kTagDims = 6;
inline bool tag_rounds(int k, int rounds) {
    return rounds >= 4 && k > kCachedDims && (k >= rounds || k >= kTagDims);
}

// Workspace of `rounds` global rounds and, with `stage`, of the subtree stage.
bool make_layout(i64 n, int k, int rounds, bool stage, Layout* out) {
    if (n < 0 || n > INT32_MAX || k < 1 || k > 65535 || rounds < 0 || rounds >= kMaxRounds)
        return false;
    Layout lay{};
    if (n <= 1) {
        *out = lay;
        return true;
    }
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    lay.rounds = rounds;
    if (rounds > 0) {
        // level l splits dimension l mod k, so the rounds use dimensions
        // 0 .. min(k, rounds)-1
        lay.kr = k < rounds ? k : rounds;
        lay.words = lay.kr + 1;
        // every dimension used again keeps its array, plus one to re-sort
        // into (a dimension used once needs its array only for its round);
        // tag rounds: their records and the subtree stage's
        lay.nbuf = stage && tag_rounds(k, rounds) ? 2 : (k < rounds ? k : 1) + 1;
        lay.tiles = (n + kPartTile - 1) / kPartTile;
        const size_t rec_bytes = (size_t)n * lay.words * sizeof(u32);
        lay.tmp0 = take(rec_bytes);  // presort pass outputs
        lay.tmp1 = take(rec_bytes);
        lay.digits = take((size_t)n);  // a presort pass's digit of each record
        lay.digits0 = take((size_t)lay.kr * n);  // the first pass's, per dimension
        lay.recs = take((size_t)lay.nbuf * rec_bytes);
        if (lay.words > kWholeWords) lay.planar0 = take(rec_bytes);
        lay.piv = take((size_t)full_nodes(rounds) * sizeof(u64));
        lay.totals = take((size_t)kRadix * sizeof(u32));
        lay.slots = take((size_t)lay.tiles * kRadix * sizeof(u32));
        lay.chunk_slots =
            take((size_t)((lay.tiles + kChunkTiles - 1) / kChunkTiles) * kRadix * sizeof(u32));
    }
    // the columns stage's: the index and at most kLocalRounds key columns
    // (none where the records carry every coordinate)
    if (stage && !stage_from_records(k, rounds)) lay.stage = take((size_t)(1 + (k < kLocalRounds ? k : kLocalRounds)) * n * sizeof(u32));
    if (stage && tag_rounds(k, rounds)) lay.tags = take((size_t)n * sizeof(u32));
    lay.total = off;
    *out = lay;
    return true;
}

// Workspace of a split-widest build: every dimension keeps an array through
// the global levels (or, with tags, the points' tags and one array of
// 16-byte records), the subtree stage reads A_0's records, and each node has
// a domain and a split dimension.
constexpr i64 kBoxChunk = 1 << 14;  // points per partial bounding box (a multiple of 4)

struct WidestLayout {
    Layout base;  // rounds = levels; records carry all k coordinates
    size_t boxes, dimtab, root_box, box_partial, level_dims;
    i64 box_chunks;
    bool by_tags;  // global levels by per-point tags (widest_tag_rounds); base.tags their array
};

int split_level(i64 n);

// Whether a split-widest build runs its global levels by per-point tags:
// with k arrays every level costs a pass over each of them, with tags a
// fixed number of passes over 16-byte records. On 4M normal points the tags
// win from k = 4 on (3.49 -> 3.22 ms at k = 4, 4.38 -> 3.38 ms at k = 5);
// k <= 3 keeps the arrays, whose LDS stage holds every dimension's order.
inline bool widest_tag_rounds(i64 n, int k) { return k > kCachedDims && split_level(n) > 0; }

bool make_layout_widest(i64 n, int k, WidestLayout* out) {
    if (n < 0 || n > INT32_MAX || k < 1 || k > 65535) return false;
    WidestLayout w{};
    if (n <= 1) {
        *out = w;
        return true;
    }
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    Layout& lay = w.base;
    lay.rounds = make_geometry(n).levels;
    lay.kr = k;
    lay.words = k + 1;
    w.by_tags = widest_tag_rounds(n, k);
    // tags: the rounds' records, then the subtree stage's planar records
    lay.nbuf = w.by_tags ? 2 : k + 1;
    lay.tiles = (n + kPartTile - 1) / kPartTile;
    const size_t rec_bytes = (size_t)n * lay.words * sizeof(u32);
    lay.tmp0 = take(rec_bytes);
    lay.tmp1 = take(rec_bytes);
    lay.digits = take((size_t)n);
    lay.digits0 = take((size_t)k * n);
    lay.recs = take((size_t)lay.nbuf * rec_bytes);
    if (lay.words > kWholeWords) lay.planar0 = take(rec_bytes);
    lay.piv = take((size_t)full_nodes(lay.rounds) * sizeof(u64));
    lay.totals = take((size_t)kRadix * sizeof(u32));
    lay.slots = take((size_t)lay.tiles * kRadix * sizeof(u32));
    lay.chunk_slots = take((size_t)((lay.tiles + kChunkTiles - 1) / kChunkTiles) * kRadix * sizeof(u32));
    w.boxes = take((size_t)n * 2 * k * sizeof(float));
    w.dimtab = take((size_t)n * sizeof(uint16_t));
    w.root_box = take((size_t)2 * k * sizeof(float));
    w.box_chunks = (n + kBoxChunk - 1) / kBoxChunk;
    w.box_partial = take((size_t)w.box_chunks * k * 2 * sizeof(float));
    w.level_dims = take((size_t)kMaxRounds * sizeof(u32));
    if (w.by_tags) lay.tags = take((size_t)n * sizeof(u32));
    lay.total = off;
    *out = w;
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

// Kernel names as the profiler prints them, per record width 0, 2, 3, 4.
int width_slot(int words) { return words == 2 ? 1 : words == 3 ? 2 : words == 4 ? 3 : 0; }
const char* const kSortScatterNames[2][4] = {
    {"k_sort_scatter<0, 0>", "k_sort_scatter<0, 2>", "k_sort_scatter<0, 3>", "k_sort_scatter<0, 4>"},
    {"k_sort_scatter<1, 0>", "k_sort_scatter<1, 2>", "k_sort_scatter<1, 3>", "k_sort_scatter<1, 4>"}};
// [round-robin, in place, split-widest, split-widest in place][width 0, 2, 3, 4]
#define KDT_PART_NAMES(kind)                                                                          \
    {{"k_part_" kind "<0>", "k_part_" kind "<2>", "k_part_" kind "<3>", "k_part_" kind "<4>"},         \
     {"k_part_" kind "_inplace<0>", "k_part_" kind "_inplace<2>", "k_part_" kind "_inplace<3>",       \
      "k_part_" kind "_inplace<4>"},                                                                  \
     {"k_part_" kind "_widest<0>", "k_part_" kind "_widest<2>", "k_part_" kind "_widest<3>",          \
      "k_part_" kind "_widest<4>"},                                                                   \
     {"k_part_" kind "_widest_inplace<0>", "k_part_" kind "_widest_inplace<2>",                       \
      "k_part_" kind "_widest_inplace<3>", "k_part_" kind "_widest_inplace<4>"}}
const char* const kPartCountNames[4][4] = KDT_PART_NAMES("count");
const char* const kPartScatterNames[4][4] = KDT_PART_NAMES("scatter");
const char* const kPartSelectNames[4][4] = KDT_PART_NAMES("select");
const char* const kPartSelectTilesNames[4][4] = KDT_PART_NAMES("select_tiles");
const char* const kPartCountBatchNames[4] = {"k_part_count_widest_batch<0>", "k_part_count_widest_batch<2>",
                                             "k_part_count_widest_batch<3>", "k_part_count_widest_batch<4>"};
const char* const kPartSelectBatchNames[4] = {"k_part_select_widest_batch<0>", "k_part_select_widest_batch<2>",
                                              "k_part_select_widest_batch<3>", "k_part_select_widest_batch<4>"};
#undef KDT_PART_NAMES

// Whether the pivots of levels l0 .. l1-1 below every tile's level-l0
// segments fit the LDS stage of the round-robin kernels. A tile of T
// positions overlapping s segments holds s - 2 of them whole, so
// s <= (T - 2) / (shortest segment) + 2; level-l0 segments hold at least
// 2^dd - 1 points (dd = L - 1 - l0 levels below), the last level one each.
bool pivots_fit(const PartArgs& a) {
    const int dd = a.geo.levels - 1 - a.l0;
    const u64 shortest = dd == 0 ? 1 : (1ull << dd) - 1;
    const u64 segs = (u64)(kPartTile - 2) / shortest + 2;
    return segs * ((1ull << (a.l1 - a.l0)) - 1) <= (u64)kPivStage;
}

// Exclusive scan of each of `rows` rows of `len` counts (and their totals):
// one workgroup a row, four times wider for rows longer than one run.
bool wide_scan(i64 len) { return len > (i64)kBlock; }
const char* scan_name(i64 len) { return wide_scan(len) ? "k_chunk_scan_wide" : "k_chunk_scan"; }
void scan_rows(u32* counts, int rows, i64 len, u32* totals, hipStream_t stream) {
    if (wide_scan(len)) k_chunk_scan_wide<<<rows, kWideScanBlock, 0, stream>>>(counts, len, totals);
    else k_chunk_scan<<<rows, kBlock, 0, stream>>>(counts, len, totals);
}

struct Launcher {
    u32* tile_counts;
    u32* chunk_counts;
    u32* totals;
    hipStream_t stream;
    Timer timer;

    // One stable pass of the presort (count, scan, scatter).
    template <int kSrc, int kW>
    void sort(SortArgs a) {
        const u64 tiles = (a.src.n + kSortTile - 1) / kSortTile;
        const u64 chunks = (tiles + kChunkTiles - 1) / kChunkTiles;
        a.tiles = (u32)tiles;
        a.chunks = chunks;
        a.tile_counts = tile_counts;
        a.chunk_counts = chunk_counts;
        a.totals = totals;
        const double n = (double)a.src.n, rec = 4.0 * a.src.words;
        timer.begin("k_sort_count", n + (double)(tiles + chunks) * kRadix * 4);
        k_sort_count<<<(unsigned)chunks, kCountBlock, 0, stream>>>(a);
        timer.end();
        timer.begin(scan_name((i64)chunks), (double)chunks * kRadix * 8);
        scan_rows(chunk_counts, kRadix, (i64)chunks, totals, stream);
        timer.end();
        // in: the rows' coordinates (and the implicit index) or the records
        const double in = kSrc == kSrcRows ? rec - 4 : rec;
        timer.begin(kSortScatterNames[kSrc][width_slot(kW)], n * (in + rec + (a.next_digits ? 1 : 0)));
        k_sort_scatter<kSrc, kW><<<xcd_grid(tiles), kSortBlock, 0, stream>>>(a);
        timer.end();
    }
    template <int kSrc>
    void sort_any(const SortArgs& a) {
        switch (a.src.words) {
            case 2: sort<kSrc, 2>(a); break;
            case 3: sort<kSrc, 3>(a); break;
            case 4: sort<kSrc, 4>(a); break;
            default: sort<kSrc, 0>(a); break;
        }
    }

    // The count kernel of a re-sort or select pass: split dimensions by
    // level (round-robin) or from the node table (split-widest); pivots
    // staged in LDS or, where a tile's may not fit, read in place.
    template <int kW>
    void count(const PartArgs& a, u64 tiles, bool widest, bool in_place) {
        const int v = (widest ? 2 : 0) + (in_place ? 1 : 0);
        timer.begin(kPartCountNames[v][width_slot(kW)], (double)a.src.n * 4.0 * a.src.words);
        const u32 g = xcd_grid(tiles);
        if (v == 0) k_part_count<kW><<<g, kBlock, 0, stream>>>(a);
        else if (v == 1) k_part_count_inplace<kW><<<g, kBlock, 0, stream>>>(a);
        else if (v == 2) k_part_count_widest<kW><<<g, kBlock, 0, stream>>>(a);
        else k_part_count_widest_inplace<kW><<<g, kBlock, 0, stream>>>(a);
        timer.end();
    }

    // One re-sort pass by tag (count, scan, scatter).
    template <int kW>
    void part(PartArgs a) {
        const u64 tiles = (a.src.n + kPartTile - 1) / kPartTile;
        a.tiles = (u32)tiles;
        a.chunk_counts = tile_counts;  // digit-major rows of per-tile counts
        const int bins = 1 << (a.l1 - a.l0);
        const double rec = 4.0 * a.src.words;
        const bool widest = a.dimtab != nullptr;  // split dimensions from the node table
        const bool in_place = kW > 0 && !pivots_fit(a);
        count<kW>(a, tiles, widest, in_place);
        timer.begin(scan_name((i64)tiles), (double)tiles * bins * 8);
        scan_rows(tile_counts, bins, (i64)tiles, nullptr, stream);
        timer.end();
        const int v = (widest ? 2 : 0) + (in_place ? 1 : 0);
        timer.begin(kPartScatterNames[v][width_slot(kW)], (double)(a.src.n + a.n_out) * rec);
        const u32 g = xcd_grid(tiles);
        if (v == 0) k_part_scatter<kW><<<g, kBlock, 0, stream>>>(a);
        else if (v == 1) k_part_scatter_inplace<kW><<<g, kBlock, 0, stream>>>(a);
        else if (v == 2) k_part_scatter_widest<kW><<<g, kBlock, 0, stream>>>(a);
        else k_part_scatter_widest_inplace<kW><<<g, kBlock, 0, stream>>>(a);
        timer.end();
    }
    void part_any(const PartArgs& a) {
        switch (a.src.words) {
            case 2: part<2>(a); break;
            case 3: part<3>(a); break;
            case 4: part<4>(a); break;
            default: part<0>(a); break;
        }
    }

    // The nodes of level a.l1 without re-sorting (count, scan, select): only
    // the tiles holding pivots are read again, at most one per node.
    template <int kW>
    void select(PartArgs a) {
        const u64 tiles = (a.src.n + kPartTile - 1) / kPartTile;
        a.tiles = (u32)tiles;
        a.chunk_counts = tile_counts;
        const int bins = 1 << (a.l1 - a.l0);
        const double rec = 4.0 * a.src.words;
        const bool widest = a.dimtab != nullptr;  // split dimensions from the node table
        const bool in_place = kW > 0 && !pivots_fit(a);
        count<kW>(a, tiles, widest, in_place);
        timer.begin(scan_name((i64)tiles), (double)tiles * bins * 8);
        scan_rows(tile_counts, bins, (i64)tiles, nullptr, stream);
        timer.end();
        // At most one node per two tiles: one workgroup per node (nodes past
        // the last leaf return), each on the tile its search finds. Else one
        // per tile, those holding pivots writing them.
        const u64 level_nodes = 1ull << a.l1, exist = (u64)a.geo.n - full_nodes(a.l1);
        const u64 nodes = level_nodes < exist ? level_nodes : exist;
        const int v = (widest ? 2 : 0) + (in_place ? 1 : 0);
        if (2 * nodes <= tiles) {
            timer.begin(kPartSelectNames[v][width_slot(kW)], (double)nodes * kPartTile * rec);
            const u32 g = (u32)nodes;
            if (v == 0) k_part_select<kW><<<g, kBlock, 0, stream>>>(a);
            else if (v == 1) k_part_select_inplace<kW><<<g, kBlock, 0, stream>>>(a);
            else if (v == 2) k_part_select_widest<kW><<<g, kBlock, 0, stream>>>(a);
            else k_part_select_widest_inplace<kW><<<g, kBlock, 0, stream>>>(a);
        } else {
            timer.begin(kPartSelectTilesNames[v][width_slot(kW)], (double)a.src.n * rec);
            const u32 g = xcd_grid(tiles);
            if (v == 0) k_part_select_tiles<kW><<<g, kBlock, 0, stream>>>(a);
            else if (v == 1) k_part_select_tiles_inplace<kW><<<g, kBlock, 0, stream>>>(a);
            else if (v == 2) k_part_select_tiles_widest<kW><<<g, kBlock, 0, stream>>>(a);
            else k_part_select_tiles_widest_inplace<kW><<<g, kBlock, 0, stream>>>(a);
        }
        timer.end();
    }
    // The select passes of one split-widest level, batched (one count, one
    // scan, one select launch) where every pass stages its pivots, walks at
    // most 6 levels (64 digit rows each: four passes fill the tile-count
    // buffer's 256 rows) and has at most one node per two tiles; else one
    // pass after another.
    template <int kW>
    void select_batch(std::vector<PartArgs> v) {
        bool ok = kW > 0 && v.size() >= 2 && v.size() <= (size_t)kMaxBatch;
        u64 max_tiles = 0;
        for (const PartArgs& a : v) {
            const u64 tiles = (a.src.n + kPartTile - 1) / kPartTile;
            const u64 level_nodes = 1ull << a.l1, exist = (u64)a.geo.n - full_nodes(a.l1);
            const u64 nodes = level_nodes < exist ? level_nodes : exist;
            ok = ok && a.l1 - a.l0 <= 6 && pivots_fit(a) && 2 * nodes <= tiles;
            max_tiles = tiles > max_tiles ? tiles : max_tiles;
        }
        if (!ok) {
            for (const PartArgs& a : v) select<kW>(a);
            return;
        }
        PartBatch b{};
        b.count = (int)v.size();
        u32 nodes_first[kMaxBatch + 1];
        double count_bytes = 0, scan_bytes = 0, select_bytes = 0;
        b.first[0] = b.rows[0] = nodes_first[0] = 0;
        for (int i = 0; i < b.count; ++i) {
            PartArgs a = v[i];
            const u64 tiles = (a.src.n + kPartTile - 1) / kPartTile;
            const u32 bins = 1u << (a.l1 - a.l0);
            const u64 level_nodes = 1ull << a.l1, exist = (u64)a.geo.n - full_nodes(a.l1);
            const u64 nodes = level_nodes < exist ? level_nodes : exist;
            a.tiles = (u32)tiles;
            a.chunk_counts = tile_counts + (u64)i * 64 * max_tiles;  // this pass's 64 rows
            b.a[i] = a;
            b.first[i + 1] = b.first[i] + xcd_grid(tiles);
            b.rows[i + 1] = b.rows[i] + bins;
            nodes_first[i + 1] = nodes_first[i] + (u32)nodes;
            const double rec = 4.0 * a.src.words;
            count_bytes += (double)a.src.n * rec;
            scan_bytes += (double)tiles * bins * 8;
            select_bytes += (double)nodes * kPartTile * rec;
        }
        timer.begin(kPartCountBatchNames[width_slot(kW)], count_bytes);
        k_part_count_widest_batch<kW><<<b.first[b.count], kBlock, 0, stream>>>(b);
        timer.end();
        timer.begin("k_chunk_scan_batch", scan_bytes);
        if (wide_scan((i64)max_tiles)) k_chunk_scan_batch<kWideScanBlock><<<b.rows[b.count], kWideScanBlock, 0, stream>>>(b);
        else k_chunk_scan_batch<kBlock><<<b.rows[b.count], kBlock, 0, stream>>>(b);
        timer.end();
        for (int i = 0; i <= b.count; ++i) b.first[i] = nodes_first[i];
        timer.begin(kPartSelectBatchNames[width_slot(kW)], select_bytes);
        k_part_select_widest_batch<kW><<<b.first[b.count], kBlock, 0, stream>>>(b);
        timer.end();
    }
    void select_batch_any(const std::vector<PartArgs>& v) {
        if (v.empty()) return;
        switch (v[0].src.words) {
            case 2: select_batch<2>(v); break;
            case 3: select_batch<3>(v); break;
            case 4: select_batch<4>(v); break;
            default: select_batch<0>(v); break;
        }
    }
    void select_any(const PartArgs& a) {
        switch (a.src.words) {
            case 2: select<2>(a); break;
            case 3: select<3>(a); break;
            case 4: select<4>(a); break;
            default: select<0>(a); break;
        }
    }
};

// Global rounds 0 .. lay.rounds-1 over all points: presorts each dimension
// at its first use, re-sorts one array per round and writes the pivots of
// every level to the pivot table (and to perm / tree when given). On return
// *last holds the array of round rounds-1 (live on that level).
kdt_status run_global(const float* pts, i64 n, int k, const Layout& lay, char* ws,
                      hipStream_t stream, Timer timer, int32_t* perm, float* tree,
                      const u32** last) {
    const int R = lay.rounds, W = lay.words;
    const Geometry geo = make_geometry(n);
    u32* tmp[2] = {(u32*)(ws + lay.tmp0), (u32*)(ws + lay.tmp1)};
    u8* digits = (u8*)(ws + lay.digits);
    u8* digits0 = (u8*)(ws + lay.digits0);
    u64* piv = (u64*)(ws + lay.piv);
    auto recs = [&](int b) { return (u32*)(ws + lay.recs) + (size_t)b * n * W; };
    Launcher launch{(u32*)(ws + lay.slots), (u32*)(ws + lay.chunk_slots), (u32*)(ws + lay.totals),
                    stream, timer};
    // Record width of A_d. With every dimension split in one round only
    // (k >= R), A_d is used in round d alone, whose walk compares
    // coordinates 0 .. d-1 (level m splits m) and whose pivots are keyed by
    // d: its records carry the keys of 0 .. d and the index. Reused arrays
    // carry every used coordinate.
    const bool narrow = k >= R;
    auto width = [&](int d) { return narrow ? d + 2 : W; };
    // Deepest walk a select may leave to the array's next pass: deeper walks
    // save re-sorts but cost more digits per count and scan, which pays off
    // with more rounds (measured best on uniform k = 3 builds: 6 up to 13
    // rounds (2^25 points), 7 at 14, 8 from 15).
    const int depth = R <= 13 ? 6 : (R == 14 ? 7 : kMaxDescent);

    // Wide records are planar; their first presort pass reads them from an
    // index-ordered planar copy of every used key built here (with the first
    // digits), the index being the position: a narrow array's first d + 1
    // planes are its keys.
    u32* planar0 = W > kWholeWords ? (u32*)(ws + lay.planar0) : nullptr;
    if (planar0) {
        timer.begin("k_planar_records", (double)n * (4.0 * k + 4.0 * W + lay.kr));
        k_planar_records<<<grid_for(n, kBlock, 1 << 16), kBlock, 0, stream>>>(pts, n, k, W, planar0, digits0);
        timer.end();
    } else {
        timer.begin(first_digits_name(pts, k), (double)n * 5.0 * lay.kr);
        launch_first_digits(pts, n, k, lay.kr, digits0, stream);
        timer.end();
    }

    int holder[kMaxRounds + 1];  // dimension whose array a buffer holds, or -1
    for (int b = 0; b <= kMaxRounds; ++b) holder[b] = -1;
    int buf_of[kMaxRounds], level_of[kMaxRounds];
    auto take = [&](int avoid) {
        for (int b = 0; b < lay.nbuf; ++b)
            if (holder[b] < 0 && b != avoid) return b;
        return -1;
    };

    for (int l = 0; l < R; ++l) {
        const int d = l % k;
        if (l < k) {
            // First use of dimension d: A_d = the points by (coordinate d,
            // index), one level-0 segment. Pass 0 reads the rows in index
            // order, pass p > 0 reads tmp[(p+1)&1]; pass p writes tmp[p&1],
            // the last one the array itself.
            const int b = take(-1);
            if (b < 0) return KDT_ERR_WORKSPACE;  // cannot happen: nbuf covers the rounds
            for (int p = 0; p < kKeyBytes; ++p) {
                SortArgs a{};
                // (records of at most four words are built from the rows)
                const bool from_planar = p == 0 && planar0 && width(d) > kWholeWords;
                a.src = RecordSource{pts, k, p == 0 ? planar0 : tmp[(p + 1) & 1], width(d), n, (u64)n, from_planar};
                a.out = p == kKeyBytes - 1 ? recs(b) : tmp[p & 1];
                a.dim = d;
                a.shift = 8 * p;
                a.digits = p == 0 ? digits0 + (size_t)d * n : digits;
                a.next_digits = p == kKeyBytes - 1 ? nullptr : digits;
                a.next_dim = d;
                a.next_shift = 8 * (p + 1);
                if (p == 0 && !from_planar) launch.sort_any<kSrcRows>(a);
                else launch.sort_any<kSrcRecords>(a);
            }
            holder[b] = d;
            buf_of[d] = b;
            level_of[d] = 0;
        }
        // Bring A_d from the tags of its last use to the level-l tags, at
        // most kMaxDescent levels per pass. The pass that reaches level l
        // only selects the pivots (the array stays where it is) when A_d is
        // not sorted again before the subtree stage, or when its next use
        // can still walk from its current level in one pass of at most
        // `depth` levels; the last global round always re-sorts (the
        // subtree stage reads its array).
        bool pivots_done = false;
        while (level_of[d] < l) {
            const int l1 = level_of[d] + kMaxDescent < l ? level_of[d] + kMaxDescent : l;
            const int next_use = l + k;
            if (l1 == l && l != R - 1 && (next_use >= R || next_use - level_of[d] <= depth)) {
                PartArgs a{};
                a.src = RecordSource{pts, k, recs(buf_of[d]), width(d), n - (i64)full_nodes(level_of[d]), (u64)n, false};
                a.k = k;
                a.l0 = level_of[d];
                a.l1 = l;
                a.dim0 = level_of[d] % k;
                a.geo = geo;
                a.s0 = level_shape(geo, a.l0);
                a.s1 = level_shape(geo, l);
                a.piv = piv;
                a.piv_out = piv;
                a.dim1 = d;
                a.s2 = level_shape(geo, l + 1);
                a.perm = perm;
                a.tree = tree;
                launch.select_any(a);
                pivots_done = true;
                break;
            }
            const int b = take(buf_of[d]);
            if (b < 0) return KDT_ERR_WORKSPACE;
            PartArgs a{};
            a.src = RecordSource{pts, k, recs(buf_of[d]), width(d), n - (i64)full_nodes(level_of[d]), (u64)n, false};
            a.out = recs(b);
            a.n_out = n - (i64)full_nodes(l1);
            a.k = k;
            a.l0 = level_of[d];
            a.l1 = l1;
            a.dim0 = level_of[d] % k;
            a.geo = geo;
            a.s0 = level_shape(geo, a.l0);
            a.s1 = level_shape(geo, a.l1);
            a.piv = piv;
            if (l1 == l) {  // this pass also fixes round l's nodes
                a.piv_out = piv;
                a.dim1 = l % k;
                a.s2 = level_shape(geo, l + 1);
                a.perm = perm;
                a.tree = tree;
                pivots_done = true;
            }
            launch.part_any(a);
            holder[buf_of[d]] = -1;
            holder[b] = d;
            buf_of[d] = b;
            level_of[d] = l1;
        }
        // Round l's nodes and their pivots (round 0 has no re-sort to do it).
        if (!pivots_done) {
            const u64 nodes = 1ull << l;
            timer.begin("k_pivots", (double)nodes * (4.0 * width(d) + 8 + (perm ? 4 : 0) + (tree ? 8.0 * k : 0)));
            k_pivots<<<(unsigned)((nodes + kBlock - 1) / kBlock), kBlock, 0, stream>>>(
                recs(buf_of[d]), width(d), (u64)n, geo, l, d, piv, pts, k, perm, tree, nullptr);
            timer.end();
        }
        // A dimension not split on again frees its array (except the last
        // round's, which the subtree stage reads).
        if (l + k >= R && l != R - 1) holder[buf_of[d]] = -1;
    }
    *last = recs(buf_of[(R - 1) % k]);
    return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
}

// Workspace of duplicate removal: two buffers of (tuple hash, index) records
// and the sort's digits and counts, one flag per point, and the
// compaction's tile counts.
struct UniqueLayout {
    Layout base;
    size_t keep, flag_counts;
    i64 flag_tiles;
};

bool make_layout_unique(i64 n, int k, UniqueLayout* out) {
    if (n < 0 || n > INT32_MAX || k < 1 || k > 65535) return false;
    UniqueLayout u{};
    if (n == 0) {
        *out = u;
        return true;
    }
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    Layout& lay = u.base;
    lay.kr = 1;
    lay.words = 2;  // (tuple hash, index)
    lay.tiles = (n + kPartTile - 1) / kPartTile;
    const size_t rec_bytes = (size_t)n * lay.words * sizeof(u32);
    lay.tmp0 = take(rec_bytes);
    lay.tmp1 = take(rec_bytes);
    lay.digits = take((size_t)n);
    lay.totals = take((size_t)kRadix * sizeof(u32));
    lay.slots = take((size_t)lay.tiles * kRadix * sizeof(u32));
    lay.chunk_slots = take((size_t)((lay.tiles + kChunkTiles - 1) / kChunkTiles) * kRadix * sizeof(u32));
    u.keep = take((size_t)n);
    u.flag_tiles = (n + kFlagTile - 1) / kFlagTile;
    u.flag_counts = take((size_t)u.flag_tiles * sizeof(u32));
    lay.total = off;
    *out = u;
    return true;
}

// Global rounds 0 .. R-1 by per-point tags (tag_rounds). Round l sorts every
// point by (node on level l, key in dimension l mod k, index): stable LSD
// passes from index order, four over the key
// and then over the node offset, so the index breaks the ties; each node's
// pivot then sits at its closed-form position (k_pivots). Records are four
// words (one vector access) whatever k is, where per-dimension arrays would each need a pass
// a round (or, with k >= R, carry the keys of every dimension a round above walks). After the last round the points are
// sorted into round R-1's order for the subtree stage: *last holds two-word
// records (position key, index), the index alone for the stage to read.
kdt_status run_global_tags(const float* pts, i64 n, int k, const Layout& lay, char* ws,
                           hipStream_t stream, Timer timer, int32_t* perm, float* tree,
                           const u32** last) {
    const int R = lay.rounds;
    const Geometry geo = make_geometry(n);
    u32* tmp[2] = {(u32*)(ws + lay.tmp0), (u32*)(ws + lay.tmp1)};
    u8* digits = (u8*)(ws + lay.digits);
    u8* digits0 = (u8*)(ws + lay.digits0);
    u64* piv = (u64*)(ws + lay.piv);
    u32* tags = (u32*)(ws + lay.tags);
    u32* planar0 = (u32*)(ws + lay.planar0);
    u32* recs0 = (u32*)(ws + lay.recs);
    u32* recs1 = recs0 + (size_t)n * lay.words;  // (two buffers of lay.words-word records)
    Launcher launch{(u32*)(ws + lay.slots), (u32*)(ws + lay.chunk_slots), (u32*)(ws + lay.totals),
                    stream, timer};
    const unsigned grid = grid_for(n, kBlock, 1 << 16);
    timer.begin("k_planar_records", (double)n * (4.0 * k + 4.0 * lay.words + lay.kr));
    k_planar_records<<<grid, kBlock, 0, stream>>>(pts, n, k, lay.words, planar0, digits0);
    timer.end();
    // one sort pass: word `word`, byte `byte` of the records, the next
    // pass's digit from (next_word, next_byte) (none: next_word < 0)
    auto pass = [&](const u32* in, int words, u32* out, int word, int byte, const u8* dig, int next_word,
                    int next_byte) {
        SortArgs a{};
        a.src = RecordSource{pts, k, in, words, n, (u64)n, false};
        a.out = out;
        a.dim = word;
        a.shift = 8 * byte;
        a.digits = dig;
        a.next_digits = next_word >= 0 ? digits : nullptr;
        a.next_dim = next_word >= 0 ? next_word : 0;
        a.next_shift = 8 * (next_byte >= 0 ? next_byte : 0);
        launch.sort_any<kSrcRecords>(a);
    };
    for (int l = 0; l < R; ++l) {
        // tags and two keys in (one key on level 0), tags and records out
        timer.begin("k_tag_level", (double)n * (l > 0 ? 32.0 : 24.0) + (l > 0 ? 8.0 * full_nodes(l) : 0));
        k_tag_level<<<grid, kBlock, 0, stream>>>(n, l, k, planar0, piv, tags, recs0);
        timer.end();
        // four key bytes, then the node offset's bytes (offsets below 2^l;
        // a fixed point's ~0 must compare above them: (l + 8) / 8 bytes)
        const int node_bytes = l == 0 ? 0 : (l + 8) / 8, passes = 4 + node_bytes;
        const u32* in = recs0;
        for (int q = 0; q < passes; ++q) {
            u32* out = tmp[q & 1];
            const int nq = q + 1;
            pass(in, 4, out, q < 4 ? 0 : 1, q < 4 ? q : q - 4, q == 0 ? digits0 + (size_t)(l % k) * n : digits,
                 nq < passes ? (nq < 4 ? 0 : 1) : -1, nq < 4 ? nq : nq - 4);
            in = out;
        }
        timer.begin("k_pivots", (double)(1ull << l) * (12.0 + 8 + (perm ? 4 : 0) + (tree ? 8.0 * k : 0)));
        k_pivots<<<(unsigned)(((1ull << l) + kBlock - 1) / kBlock), kBlock, 0, stream>>>(
            in, 4, (u64)n, geo, l, 0, piv, pts, k, perm, tree, nullptr);
        timer.end();
    }
    timer.begin("k_tag_subtrees", (double)n * (4.0 + 4 + 8 + 1) + 8.0 * full_nodes(R));
    k_tag_subtrees<<<grid, kBlock, 0, stream>>>(n, R, k, planar0, piv, tags, recs0, digits);
    timer.end();
    // position keys below 3 * 2^(R-1) < 2^(R+1), ~0 above them
    const int key_bytes = (R + 1 + 7) / 8;
    const u32* in = recs0;
    for (int q = 0; q < key_bytes; ++q) {
        u32* out = q == key_bytes - 1 ? recs1 : tmp[q & 1];
        pass(in, 2, out, 0, q, digits, q + 1 < key_bytes ? 0 : -1, q + 1);
        in = out;
    }
    *last = recs1;
    return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
}

// Duplicate removal: the points' (tuple hash, index) records sorted by hash
// with 4 stable LSD radix passes (equal tuples then sit together, in index
// order), the run heads with exact comparisons inside equal-hash runs, then
// the compaction in index order.
kdt_status run_unique(const float* pts, i64 n, int k, const UniqueLayout& ul, char* ws,
                      hipStream_t stream, Timer timer, int32_t* keep_out, int64_t* count_out) {
    const Layout& lay = ul.base;
    const int W = lay.words;
    u32* tmp[2] = {(u32*)(ws + lay.tmp0), (u32*)(ws + lay.tmp1)};
    u8* digits = (u8*)(ws + lay.digits);
    u32* totals = (u32*)(ws + lay.totals);
    u8* keep = (u8*)(ws + ul.keep);
    u32* flag_counts = (u32*)(ws + ul.flag_counts);
    Launcher launch{(u32*)(ws + lay.slots), (u32*)(ws + lay.chunk_slots), totals, stream, timer};

    timer.begin("k_hash_records", (double)n * (4.0 * k + 9));
    k_hash_records<<<grid_for(n, kBlock, 1 << 16), kBlock, 0, stream>>>(pts, n, k, tmp[1], digits);
    timer.end();
    // (hash, index) records by hash, stably from index order: 4 LSD passes,
    // tmp[1] -> tmp[0] -> tmp[1] -> tmp[0] -> tmp[1]
    const u32* sorted = nullptr;
    for (int p = 0; p < kKeyBytes; ++p) {
        SortArgs a{};
        a.src = RecordSource{pts, k, tmp[(p + 1) & 1], W, n, (u64)n, false};
        a.out = tmp[p & 1];
        a.dim = 0;
        a.shift = 8 * p;
        a.digits = digits;
        a.next_digits = p + 1 < kKeyBytes ? digits : nullptr;
        a.next_dim = 0;
        a.next_shift = 8 * (p + 1);
        launch.sort_any<kSrcRecords>(a);
        sorted = a.out;
    }
    timer.begin("k_keep_all", (double)n);
    k_keep_all<<<grid_for((n + 3) / 4, kBlock, 1 << 16), kBlock, 0, stream>>>(reinterpret_cast<u32*>(keep),
                                                                             (n + 3) / 4);
    timer.end();
    timer.begin("k_unique_mark", (double)n * 4.0 * W);
    k_unique_mark<<<grid_for(n, kBlock, 1 << 16), kBlock, 0, stream>>>(sorted, n, pts, k, keep);
    timer.end();
    const i64 T = ul.flag_tiles;
    timer.begin("k_flag_count", (double)n + 4.0 * T);
    k_flag_count<<<(unsigned)T, kBlock, 0, stream>>>(keep, n, flag_counts);
    timer.end();
    timer.begin("k_chunk_scan", (double)T * 8);
    k_chunk_scan<<<1, kBlock, 0, stream>>>(flag_counts, T, totals);
    timer.end();
    timer.begin("k_flag_compact", (double)n * 5.0);
    k_flag_compact<<<(unsigned)T, kBlock, 0, stream>>>(keep, n, flag_counts, totals, keep_out, count_out);
    timer.end();
    return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
}

// A split-widest-dimension build ([W], split-widest-dimension section): the
// root domain and dimension first; every dimension's array presorted; then
// level by level, every array re-sorted by the new tags (one pass of one
// level), each fixing the nodes of the level that split its dimension, and
// the next level's domains and dimensions from the pivots just fixed. The
// last level's pass places the leaves.
// Levels 0 .. lds_from-1 as global passes (every level when lds_from = L),
// then, if lds_from < L, the subtrees of level lds_from in LDS.
kdt_status run_widest(const float* pts, i64 n, int k, const WidestLayout& wl, char* ws,
                      hipStream_t stream, Timer timer, int32_t* perm, float* tree,
                      int32_t* dims_out, int lds_from) {
    const Layout& lay = wl.base;
    const int L = lay.rounds, W = lay.words;
    const Geometry geo = make_geometry(n);
    u32* tmp[2] = {(u32*)(ws + lay.tmp0), (u32*)(ws + lay.tmp1)};
    u8* digits = (u8*)(ws + lay.digits);
    u8* digits0 = (u8*)(ws + lay.digits0);
    u64* piv = (u64*)(ws + lay.piv);
    float* boxes = (float*)(ws + wl.boxes);
    uint16_t* dimtab = (uint16_t*)(ws + wl.dimtab);
    float* root_box = (float*)(ws + wl.root_box);
    float* partial = (float*)(ws + wl.box_partial);
    // each level's split dimensions, for skipping selects with no pivot to
    // find (dimension masks need k <= 32)
    u32* level_dims = k <= 32 ? (u32*)(ws + wl.level_dims) : nullptr;
    auto recs = [&](int b) { return (u32*)(ws + lay.recs) + (size_t)b * n * W; };
    Launcher launch{(u32*)(ws + lay.slots), (u32*)(ws + lay.chunk_slots), (u32*)(ws + lay.totals),
                    stream, timer};
    auto level = [&](int l) {
        const u64 nodes = 1ull << l;
        timer.begin("k_widest_level", (double)nodes * (16.0 * k + 10 + (dims_out ? 4 : 0)));
        k_widest_level<<<(unsigned)((nodes + kBlock - 1) / kBlock), kBlock, 0, stream>>>(
            geo, l, k, piv, root_box, boxes, dimtab, dims_out, level_dims);
        timer.end();
    };

    if (level_dims) {
        timer.begin("k_zero", 4.0 * kMaxRounds);
        k_zero<<<1, kBlock, 0, stream>>>(level_dims, kMaxRounds);
        timer.end();
    }
    static const char* const kBoxNames[5] = {"k_box_partial", "k_box_partial4<1>", "k_box_partial4<2>",
                                             "k_box_partial4<3>", "k_box_partial4<4>"};
    timer.begin(kBoxNames[first_digits_vec(pts, k) ? k : 0], (double)n * 4.0 * k);
    if (first_digits_vec(pts, k) && k == 1) k_box_partial4<1><<<(unsigned)wl.box_chunks, kBlock, 0, stream>>>(pts, n, kBoxChunk, partial);
    else if (first_digits_vec(pts, k) && k == 2) k_box_partial4<2><<<(unsigned)wl.box_chunks, kBlock, 0, stream>>>(pts, n, kBoxChunk, partial);
    else if (first_digits_vec(pts, k) && k == 3) k_box_partial4<3><<<(unsigned)wl.box_chunks, kBlock, 0, stream>>>(pts, n, kBoxChunk, partial);
    else if (first_digits_vec(pts, k) && k == 4) k_box_partial4<4><<<(unsigned)wl.box_chunks, kBlock, 0, stream>>>(pts, n, kBoxChunk, partial);
    else k_box_partial<<<dim3((unsigned)wl.box_chunks, (unsigned)k), kBlock, 0, stream>>>(pts, n, k, kBoxChunk, partial);
    timer.end();
    timer.begin("k_box_final", (double)wl.box_chunks * k * 8.0 + 8.0 * k);
    k_box_final<<<(unsigned)k, kBlock, 0, stream>>>(partial, wl.box_chunks, k, root_box);
    timer.end();
    level(0);

    auto subtrees = [&](const u32* arrival) {
        WidestSubtreeArgs sa{};
        sa.pts = pts;
        sa.n = n;
        sa.k = k;
        sa.l0 = lds_from;
        sa.geo = geo;
        sa.recs = arrival;
        sa.boxes = boxes;
        sa.dimtab = dimtab;
        sa.perm = perm;
        sa.tree = tree;
        sa.dims_out = dims_out;
        const double below = (double)(n - (i64)full_nodes(lds_from));
        static const char* const kNames[kCachedDims + 2] = {"", "k_subtree_widest<1>", "k_subtree_widest<2>",
                                                            "k_subtree_widest<3>", "k_subtree_widest_cols"};
        // records (or rows) in and out; each node's domain written (the last
        // level's excepted) and read once by its children's pivot thread
        timer.begin(kNames[k <= kCachedDims ? k : kCachedDims + 1],
                    below * (4.0 * W + 4 + (tree ? 4.0 * k : 0) + (dims_out ? 4 : 0) + 2 * 8.0 * k));
        const unsigned subtrees_n = (unsigned)(1ull << lds_from);
        if (k == 1) k_subtree_widest<1><<<subtrees_n, kLocalBlock, 0, stream>>>(sa);
        else if (k == 2) k_subtree_widest<2><<<subtrees_n, kLocalBlock, 0, stream>>>(sa);
        else if (k == 3) k_subtree_widest<3><<<subtrees_n, kLocalBlock, 0, stream>>>(sa);
        else k_subtree_widest_cols<<<subtrees_n, kLocalBlock, 0, stream>>>(sa);
        timer.end();
    };
    if (lds_from == 0) {  // the whole tree is one subtree, from the rows
        subtrees(nullptr);
        return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
    }
    if (wl.by_tags) {
        // Levels 0 .. lds_from-1 by per-point tags: each level sorts every
        // point by (node, key in the node's split dimension, index) with
        // stable LSD passes from index order and takes the pivots at their
        // closed-form positions; then the points are sorted by their node on
        // level lds_from and written as the stage's planar records.
        u32* planar0 = (u32*)(ws + lay.planar0);
        u32* tags = (u32*)(ws + lay.tags);
        u32* recs0 = recs(0);
        u32* recs1 = recs(1);
        const unsigned grid = grid_for(n, kBlock, 1 << 16);
        timer.begin("k_planar_records", (double)n * (4.0 * k + 4.0 * W + k));
        k_planar_records<<<grid, kBlock, 0, stream>>>(pts, n, k, W, planar0, digits0);
        timer.end();
        auto pass = [&](const u32* in, int words, u32* out, int word, int byte, int next_word, int next_byte) {
            SortArgs a{};
            a.src = RecordSource{pts, k, in, words, n, (u64)n, false};
            a.out = out;
            a.dim = word;
            a.shift = 8 * byte;
            a.digits = digits;
            a.next_digits = next_word >= 0 ? digits : nullptr;
            a.next_dim = next_word >= 0 ? next_word : 0;
            a.next_shift = 8 * (next_byte >= 0 ? next_byte : 0);
            launch.sort_any<kSrcRecords>(a);
        };
        for (int l = 0; l < lds_from; ++l) {
            timer.begin("k_wtag_level", (double)n * (l > 0 ? 33.0 : 25.0) + (l > 0 ? 10.0 * full_nodes(l) : 0));
            k_wtag_level<<<grid, kBlock, 0, stream>>>(n, l, planar0, piv, dimtab, tags, recs0, digits);
            timer.end();
            const int node_bytes = l == 0 ? 0 : (l + 8) / 8, passes = 4 + node_bytes;
            const u32* in = recs0;
            for (int q = 0; q < passes; ++q) {
                u32* out = tmp[q & 1];
                const int nq = q + 1;
                pass(in, 4, out, q < 4 ? 0 : 1, q < 4 ? q : q - 4, nq < passes ? (nq < 4 ? 0 : 1) : -1,
                     nq < 4 ? nq : nq - 4);
                in = out;
            }
            timer.begin("k_pivots", (double)(1ull << l) * (16.0 + 8 + (perm ? 4 : 0) + (tree ? 8.0 * k : 0)));
            k_pivots<<<(unsigned)(((1ull << l) + kBlock - 1) / kBlock), kBlock, 0, stream>>>(
                in, 4, (u64)n, geo, l, 0, piv, pts, k, perm, tree, nullptr);
            timer.end();
            level(l + 1);  // (lds_from < L)
        }
        timer.begin("k_wtag_subtrees", (double)n * (4.0 + 4 + 2 + 8 + 1));
        k_wtag_subtrees<<<grid, kBlock, 0, stream>>>(n, lds_from, planar0, piv, dimtab, tags, recs0, digits);
        timer.end();
        // node offsets below 2^lds_from, ~0 above them
        const int key_bytes = (lds_from + 8) / 8;
        const u32* in = recs0;
        for (int q = 0; q < key_bytes; ++q) {
            u32* out = tmp[q & 1];
            pass(in, 2, out, 0, q, q + 1 < key_bytes ? 0 : -1, q + 1);
            in = out;
        }
        const i64 live = n - (i64)full_nodes(lds_from);
        timer.begin("k_wtag_planar", (double)live * (4.0 + 8.0 * k + 4));
        k_wtag_planar<<<grid_for(live, kBlock, 1 << 16), kBlock, 0, stream>>>(live, n, k, pts, in, recs1);
        timer.end();
        subtrees(recs1);
        return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
    }

    u32* planar0 = W > kWholeWords ? (u32*)(ws + lay.planar0) : nullptr;
    if (planar0) {
        timer.begin("k_planar_records", (double)n * (4.0 * k + 4.0 * W + k));
        k_planar_records<<<grid_for(n, kBlock, 1 << 16), kBlock, 0, stream>>>(pts, n, k, W, planar0, digits0);
        timer.end();
    } else {
        timer.begin(first_digits_name(pts, k), (double)n * 5.0 * k);
        launch_first_digits(pts, n, k, k, digits0, stream);
        timer.end();
    }
    // A_d in buffer d, by (coordinate d, index): the order of level 0.
    for (int d = 0; d < k; ++d)
        for (int p = 0; p < kKeyBytes; ++p) {
            SortArgs a{};
            a.src = RecordSource{pts, k, p == 0 ? planar0 : tmp[(p + 1) & 1], W, n, (u64)n, false};
            a.out = p == kKeyBytes - 1 ? recs(d) : tmp[p & 1];
            a.dim = d;
            a.shift = 8 * p;
            a.digits = p == 0 ? digits0 + (size_t)d * n : digits;
            a.next_digits = p == kKeyBytes - 1 ? nullptr : digits;
            a.next_dim = d;
            a.next_shift = 8 * (p + 1);
            if (p == 0 && !planar0) launch.sort_any<kSrcRows>(a);
            else launch.sort_any<kSrcRecords>(a);
        }
    std::vector<int> buffer(k);
    for (int d = 0; d < k; ++d) buffer[d] = d;
    int spare = k;
    // The root's pivot, from the array of its dimension.
    for (int d = 0; d < k; ++d) {
        timer.begin("k_pivots", 4.0 * W + 8 + (perm ? 4 : 0) + (tree ? 8.0 * k : 0));
        k_pivots<<<1, kBlock, 0, stream>>>(recs(buffer[d]), W, (u64)n, geo, 0, d, piv, pts, k, perm, tree, dimtab);
        timer.end();
    }
    if (L > 1) level(1);
    // Every level finds each array's nodes' pivots in that array. An array
    // is re-sorted to the level only where that is cheaper than a select:
    // not where no later pass reads it (the last level; on the last global
    // level, every array but A_0, which the subtree stage reads), and not
    // while the level has few nodes for the tiles (2^l <= tiles / 2) and
    // the array's next walk stays within kSelectDepth levels.
    const u64 tiles = ((u64)n + kPartTile - 1) / kPartTile;
    std::vector<int> level_of(k, 0);
    for (int l = 1; l < lds_from; ++l) {
        std::vector<PartArgs> selects;  // this level's, launched together after the re-sorts
        for (int d = 0; d < k; ++d) {
            PartArgs a{};
            a.src = RecordSource{pts, k, recs(buffer[d]), W, n - (i64)full_nodes(level_of[d]), (u64)n, false};
            a.out = recs(spare);
            a.n_out = n - (i64)full_nodes(l);
            a.k = k;
            a.l0 = level_of[d];
            a.l1 = l;
            a.dim0 = 0;
            a.geo = geo;
            a.s0 = level_shape(geo, level_of[d]);
            a.s1 = level_shape(geo, l);
            a.piv = piv;
            a.piv_out = piv;
            a.dim1 = d;
            if (l + 1 < L) a.s2 = level_shape(geo, l + 1);
            a.perm = perm;
            a.tree = tree;
            a.dimtab = dimtab;
            a.array_dim = d;
            a.leaf_level = l == L - 1;
            const bool unread = lds_from == L ? l == L - 1 : l == lds_from - 1 && d != 0;
            const bool select = unread || ((2ull << l) <= tiles && l + 1 - level_of[d] <= kSelectDepth);
            if (select) {
                a.level_dims = level_dims;
                selects.push_back(a);
            } else {
                launch.part_any(a);
                std::swap(buffer[d], spare);
                level_of[d] = l;
            }
        }
        launch.select_batch_any(selects);
        if (l + 1 < L) level(l + 1);
    }
    if (lds_from < L) {
        // A_0 to level lds_from (no pivots: the subtree stage fixes that
        // level's nodes), so that each subtree's records are one range.
        PartArgs a{};
        a.src = RecordSource{pts, k, recs(buffer[0]), W, n - (i64)full_nodes(level_of[0]), (u64)n, false};
        a.out = recs(spare);
        a.n_out = n - (i64)full_nodes(lds_from);
        a.k = k;
        a.l0 = level_of[0];
        a.l1 = lds_from;
        a.geo = geo;
        a.s0 = level_shape(geo, level_of[0]);
        a.s1 = level_shape(geo, lds_from);
        if (lds_from + 1 < L) a.s2 = level_shape(geo, lds_from + 1);
        a.piv = piv;
        a.dimtab = dimtab;
        launch.part_any(a);
        std::swap(buffer[0], spare);
        subtrees(recs(buffer[0]));
    }
    return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
}

kdt_status validate(const float* pts, i64 n, int k, const void* out0, size_t out0_bytes,
                    const void* out1, size_t out1_bytes, void* ws, size_t ws_bytes,
                    const Layout& lay) {
    if (n == 0) return KDT_OK;
    if (!pts || !out0) return KDT_ERR_INVALID_ARG;
    const size_t pts_bytes = (size_t)n * k * sizeof(float);
    if (ranges_overlap(pts, pts_bytes, out0, out0_bytes) ||
        ranges_overlap(pts, pts_bytes, out1, out1_bytes) ||
        ranges_overlap(out0, out0_bytes, out1, out1_bytes))
        return KDT_ERR_INVALID_ARG;
    if (lay.total > 0) {
        if (!ws || ws_bytes < lay.total || ((uintptr_t)ws & 255)) return KDT_ERR_WORKSPACE;
        if (ranges_overlap(ws, lay.total, pts, pts_bytes) ||
            ranges_overlap(ws, lay.total, out0, out0_bytes) ||
            ranges_overlap(ws, lay.total, out1, out1_bytes))
            return KDT_ERR_INVALID_ARG;
    }
    return KDT_OK;
}

bool valid_size(i64 n, int k) { return n >= 0 && n <= INT32_MAX && k >= 1 && k <= 65535; }

// First level whose subtrees all fit one workgroup (the leftmost subtree of
// a level is the largest one).
int split_level(i64 n) {
    if (n <= 1) return 0;
    const Geometry g = make_geometry(n);
    int l = 0;
    while (subtree_size(g, full_nodes(l)) > (u64)kLocalMax) ++l;
    return l;
}

kdt_status build_impl(const float* points, int64_t N, int32_t k, int32_t* perm_out,
                      float* tree_out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream, Timer timer) {
    if (!valid_size(N, k)) return KDT_ERR_INVALID_ARG;
    const int l0 = split_level(N);
    Layout lay;
    if (!make_layout(N, k, l0, true, &lay)) return KDT_ERR_INVALID_ARG;
    const size_t perm_bytes = (size_t)N * sizeof(int32_t);
    const size_t tree_bytes = tree_out ? (size_t)N * k * sizeof(float) : 0;
    kdt_status st = validate(points, N, k, perm_out, perm_bytes, tree_out, tree_bytes, workspace,
                             workspace_bytes, lay);
    if (st != KDT_OK || N == 0) return st;
    if (N == 1) {
        timer.begin("k_single", 4.0 + (tree_out ? 8.0 * k : 0));
        k_single<<<1, 64, 0, stream>>>(points, k, perm_out, tree_out);
        timer.end();
        return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
    }
    const Geometry geo = make_geometry(N);
    const u32* recs = nullptr;
    const bool by_tags = tag_rounds(k, l0);
    if (l0 > 0) {
        st = by_tags ? run_global_tags(points, N, k, lay, (char*)workspace, stream, timer, perm_out, tree_out, &recs)
                     : run_global(points, N, k, lay, (char*)workspace, stream, timer, perm_out, tree_out, &recs);
        if (st != KDT_OK) return st;
    }
    SubtreeArgs sa{};
    sa.pts = points;
    sa.n = N;
    sa.k = k;
    sa.l0 = l0;
    sa.geo = geo;
    sa.recs = recs;
    sa.words = by_tags ? 2 : lay.words;
    sa.index_only = by_tags;
    sa.plane = (u64)N;
    // records that carry every coordinate (then lay.words == k + 1) are read
    // in place, else staged
    const bool from_recs = stage_from_records(k, l0);
    sa.stage = from_recs ? nullptr : (u32*)((char*)workspace + lay.stage);
    sa.perm = perm_out;
    sa.tree = tree_out;
    const i64 below = N - (i64)full_nodes(l0);  // points in the level-l0 subtrees
    const double row = 4.0 * k;
    // per point: records: the record in, perm and the row out. Columns: the
    // index and the keys of the (at most kLocalRounds) dimensions the rounds
    // split in, staged and read back, perm out and the row copied.
    const int local_rounds = make_geometry((i64)subtree_size(geo, full_nodes(l0))).levels - 1;
    const int used = local_rounds < k ? local_rounds : k;
    const double cols = 4.0 * (1 + used) * 3 + 4 + (tree_out ? 2 * row : 0);
    static const char* const kRecNames[kCachedDims + 1] = {"", "k_subtree_recs<1>", "k_subtree_recs<2>",
                                                           "k_subtree_recs<3>"};
    timer.begin(from_recs ? kRecNames[k] : "k_subtree_cols",
                (double)below * (from_recs ? 4.0 * lay.words + 4 + (tree_out ? row : 0) : cols));
    const unsigned subtrees = (unsigned)(1ull << l0);
    if (from_recs && k == 1) k_subtree_recs<1><<<subtrees, kLocalBlock, 0, stream>>>(sa);
    else if (from_recs && k == 2) k_subtree_recs<2><<<subtrees, kLocalBlock, 0, stream>>>(sa);
    else if (from_recs) k_subtree_recs<3><<<subtrees, kLocalBlock, 0, stream>>>(sa);
    else k_subtree_cols<<<subtrees, kLocalBlock, 0, stream>>>(sa);
    timer.end();
    return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
}

kdt_status build_widest_impl(const float* points, int64_t N, int32_t k, int32_t* perm_out,
                             float* tree_out, int32_t* dims_out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream, Timer timer) {
    WidestLayout wl;
    if (!valid_size(N, k) || !make_layout_widest(N, k, &wl)) return KDT_ERR_INVALID_ARG;
    const size_t perm_bytes = (size_t)N * sizeof(int32_t);
    const size_t tree_bytes = tree_out ? (size_t)N * k * sizeof(float) : 0;
    const size_t dims_bytes = dims_out ? (size_t)N * sizeof(int32_t) : 0;
    kdt_status st = validate(points, N, k, perm_out, perm_bytes, tree_out, tree_bytes, workspace,
                             workspace_bytes, wl.base);
    if (st != KDT_OK) return st;
    if (dims_out && N > 0) {
        const size_t pts_bytes = (size_t)N * k * sizeof(float);
        if (ranges_overlap(dims_out, dims_bytes, points, pts_bytes) ||
            ranges_overlap(dims_out, dims_bytes, perm_out, perm_bytes) ||
            ranges_overlap(dims_out, dims_bytes, tree_out, tree_bytes) ||
            ranges_overlap(dims_out, dims_bytes, workspace, wl.base.total))
            return KDT_ERR_INVALID_ARG;
    }
    if (N == 0) return KDT_OK;
    if (N == 1) {  // one point: its domain has no extent, so dimension 0
        timer.begin("k_single", 4.0 + (tree_out ? 8.0 * k : 0));
        k_single<<<1, 64, 0, stream>>>(points, k, perm_out, tree_out);
        timer.end();
        if (dims_out) k_zero<<<1, kBlock, 0, stream>>>(reinterpret_cast<u32*>(dims_out), 1);
        return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
    }
    // Subtrees of at most kLocalMax points finish in LDS.
    const int lds_from = split_level(N);
    return run_widest(points, N, k, wl, (char*)workspace, stream, timer, perm_out, tree_out, dims_out,
                      lds_from);
}

kdt_status unique_impl(const float* points, int64_t N, int32_t k, int32_t* keep_out, int64_t* count_out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream, Timer timer) {
    UniqueLayout ul;
    if (!valid_size(N, k) || !make_layout_unique(N, k, &ul)) return KDT_ERR_INVALID_ARG;
    if (!count_out) return KDT_ERR_INVALID_ARG;
    const size_t keep_bytes = (size_t)N * sizeof(int32_t);
    kdt_status st = validate(points, N, k, keep_out, keep_bytes, count_out, sizeof(int64_t), workspace,
                             workspace_bytes, ul.base);
    if (st != KDT_OK) return st;
    if (N == 0) {
        k_zero<<<1, kBlock, 0, stream>>>(reinterpret_cast<u32*>(count_out), 2);
        return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
    }
    return run_unique(points, N, k, ul, (char*)workspace, stream, timer, keep_out, count_out);
}

// Runs `build` with a HIP event pair around every kernel, synchronises and
// fills *profile.
template <typename Build>
kdt_status run_profiled(hipStream_t stream, kdt_profile* profile, Build build) {
    if (!profile) return KDT_ERR_INVALID_ARG;
    Profiler* prof = new Profiler();
    prof->stream = stream;
    kdt_status st = build(Timer{prof});
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
    if (prof->failed && st == KDT_OK) st = KDT_ERR_HIP;  // event API failure or too many kinds
    delete prof;
    return st;
}

}  // namespace

// ------------------------------------------ allocation-free entry point
// kdt_build_static runs kdt_build with this file-scope device array as its
// workspace, for callers that cannot allocate. Each device holds its own
// copy for the life of the process. In host code `scratch` names a host-side
// stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[KDT_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call per device).
kdt_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDT_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDT_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KDT_OK;
}

}  // namespace

extern "C" {

size_t kdt_workspace_size(int64_t N, int32_t k) {
    if (!valid_size(N, k)) return 0;
    Layout lay;
    if (!make_layout(N, k, split_level(N), true, &lay)) return 0;
    return lay.total;
}

size_t kdt_debug_workspace_size(int64_t N, int32_t k, int32_t rounds) {
    if (!valid_size(N, k) || N <= 1) return 0;
    if (rounds < 0 || rounds > make_geometry(N).levels - 1) return 0;
    Layout lay;
    if (!make_layout(N, k, rounds, false, &lay)) return 0;
    return lay.total;
}

kdt_status kdt_build(const float* points, int64_t N, int32_t k, int32_t* perm_out,
                     float* tree_out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    return build_impl(points, N, k, perm_out, tree_out, workspace, workspace_bytes, stream,
                      Timer{nullptr});
}

kdt_status kdt_build_static(const float* points, int64_t N, int32_t k, int32_t* perm_out,
                            float* tree_out, hipStream_t stream) {
    if (!valid_size(N, k)) return KDT_ERR_INVALID_ARG;
    if (kdt_workspace_size(N, k) > KDT_STATIC_SCRATCH_BYTES) return KDT_ERR_TOO_LARGE;
    void* ws = nullptr;
    if (N > 1) {
        const kdt_status st = scratch_address(&ws);
        if (st != KDT_OK) return st;
    }
    return build_impl(points, N, k, perm_out, tree_out, ws, KDT_STATIC_SCRATCH_BYTES, stream,
                      Timer{nullptr});
}

kdt_status kdt_build_profiled(const float* points, int64_t N, int32_t k, int32_t* perm_out,
                              float* tree_out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, kdt_profile* profile) {
    return run_profiled(stream, profile, [&](Timer timer) {
        return build_impl(points, N, k, perm_out, tree_out, workspace, workspace_bytes, stream, timer);
    });
}

size_t kdt_unique_workspace_size(int64_t N, int32_t k) {
    UniqueLayout ul;
    if (!valid_size(N, k) || !make_layout_unique(N, k, &ul)) return 0;
    return ul.base.total;
}

kdt_status kdt_unique(const float* points, int64_t N, int32_t k, int32_t* keep_out, int64_t* count_out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return unique_impl(points, N, k, keep_out, count_out, workspace, workspace_bytes, stream, Timer{nullptr});
}

kdt_status kdt_unique_profiled(const float* points, int64_t N, int32_t k, int32_t* keep_out,
                               int64_t* count_out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream, kdt_profile* profile) {
    return run_profiled(stream, profile, [&](Timer timer) {
        return unique_impl(points, N, k, keep_out, count_out, workspace, workspace_bytes, stream, timer);
    });
}

size_t kdt_workspace_size_widest(int64_t N, int32_t k) {
    WidestLayout wl;
    if (!valid_size(N, k) || !make_layout_widest(N, k, &wl)) return 0;
    return wl.base.total;
}

kdt_status kdt_build_widest(const float* points, int64_t N, int32_t k, int32_t* perm_out,
                            float* tree_out, int32_t* dims_out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    return build_widest_impl(points, N, k, perm_out, tree_out, dims_out, workspace, workspace_bytes,
                             stream, Timer{nullptr});
}

kdt_status kdt_build_widest_profiled(const float* points, int64_t N, int32_t k, int32_t* perm_out,
                                     float* tree_out, int32_t* dims_out, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream,
                                     kdt_profile* profile) {
    return run_profiled(stream, profile, [&](Timer timer) {
        return build_widest_impl(points, N, k, perm_out, tree_out, dims_out, workspace,
                                 workspace_bytes, stream, timer);
    });
}

kdt_status kdt_debug_tags(const float* points, int64_t N, int32_t k, int32_t rounds,
                          uint32_t* tags_out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    if (!valid_size(N, k)) return KDT_ERR_INVALID_ARG;
    if (N == 0) return KDT_OK;
    const int max_rounds = make_geometry(N).levels - 1;
    if (rounds < 0 || rounds > max_rounds) return KDT_ERR_INVALID_ARG;
    Layout lay;
    if (!make_layout(N, k, rounds, false, &lay)) return KDT_ERR_INVALID_ARG;
    const size_t tag_bytes = (size_t)N * sizeof(u32);
    kdt_status st = validate(points, N, k, tags_out, tag_bytes, nullptr, 0, workspace,
                             workspace_bytes, lay);
    if (st != KDT_OK) return st;
    const int grid = grid_for(N, kBlock * 4, 8192);
    if (rounds == 0) {
        k_zero<<<grid, kBlock, 0, stream>>>(tags_out, N);
        return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_HIP;
    }
    const u32* last = nullptr;
    st = run_global(points, N, k, lay, (char*)workspace, stream, Timer{nullptr}, nullptr, nullptr,
                    &last);
    if (st != KDT_OK) return st;
    k_descend_tags<<<grid, kBlock, 0, stream>>>(points, N, k, rounds,
                                               (const u64*)((char*)workspace + lay.piv), tags_out);
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

int64_t kdt_closed_live_segment(int64_t N, int32_t l, int64_t p) {
    if (N <= 0 || N > INT32_MAX) return -1;
    const Geometry g = make_geometry(N);
    if (l < 0 || l >= g.levels || p < 0 || p >= N - (int64_t)full_nodes(l)) return -1;
    return (int64_t)live_segment(g, (u64)p, l);
}

int64_t kdt_closed_bin_prefix(int64_t N, int32_t l1, int32_t delta, int64_t j0, int64_t b) {
    if (N <= 0 || N > INT32_MAX) return -1;
    const Geometry g = make_geometry(N);
    if (l1 < 0 || l1 >= g.levels || delta < 0 || delta > l1 || delta > kMaxDescent) return -1;
    if (j0 < 0 || j0 > (int64_t)(1ull << (l1 - delta)) || b < 0 || b >= (int64_t)(1ull << delta))
        return -1;
    return (int64_t)bin_prefix(g, (u64)j0, (u32)b, l1, delta);
}

void kdt_closed_float_keys(const uint32_t* bits, int64_t n, uint32_t* keys_out) {
    if (n <= 0 || !bits || !keys_out) return;
    for (int64_t i = 0; i < n; ++i) keys_out[i] = float_key(bits[i]);
}

const char* kdt_status_string(kdt_status status) {
    switch (status) {
        case KDT_OK: return "ok";
        case KDT_ERR_INVALID_ARG: return "invalid argument";
        case KDT_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case KDT_ERR_HIP: return "HIP kernel launch failed";
        case KDT_ERR_TOO_LARGE: return "N and k need more workspace than the static scratch array holds";
    }
    return "unknown status";
}

}  // extern "C"
