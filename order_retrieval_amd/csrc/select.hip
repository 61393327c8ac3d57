// select.hip -- exact causal top-k selection on the Z-order line.
//
// "ZETA: Leveraging Z-order Curves for Efficient Top-k Attention", rebuttal page, answers
// W3/A3 and W2/A2 ("Clarification"): keys are sorted on the 1-D Z-order line and a query
// finds its neighbours by binary search for its insertion position and a window around
// it; summary page ("Approach"): sorting and chunking lets every query of a causal
// sequence retrieve its top-k in parallel.
//
// Exact form computed here: for query i, the k keys j <= i with the smallest
// (|zq_i - zk_j|, j).  The prefix [0, i] is split into the aligned power-of-two blocks
// given by the set bits of i+1 (largest first); each block is a sorted run of the
// merge-sort tree.  In a run, the keys with code >= zq ordered by (code, j) start at the
// insertion position p of the asc tree; the keys with code < zq ordered by (-code, j) end
// just before p in the desc tree (same p: both trees hold the same codes).  Any key of the
// global top-k is among the first k of one of those two walks in its own run, so merging
// the first k of every walk gives the exact answer.
//
// The running top-K (K = next power of two >= k) of a query is a sorted list of packed keys
// (|dz| << 32) | j spread over L consecutive lanes of a wavefront (L = 4 for K = 16, 8 for
// K = 32 and 64, a whole 16-lane row for K = 128 and 256: 4 to 16 entries per lane, so more
// wavefronts fit and each query's merge work is spread; L = 1 below K = 16).  A
// walk's K candidates are merged with one bitonic step: elementwise min against the
// reversed candidates (each lane loads its own contiguous block of the walk) leaves a
// bitonic sequence of the K smallest, which log2(K) compare-exchange stages sort; the stages
// whose stride spans lanes exchange values with DPP quad permutes (lanes 4 or 8 apart: a
// ds_swizzle, which moves data between lanes without touching LDS memory; broadcasts inside
// a group of 8 are ds_swizzles too, inside a 16-lane row DPP row broadcasts).  A walk whose first
// candidate cannot beat the current K-th is skipped, decided from values the search already
// holds.  The runs are taken in groups: with several lanes per query each lane
// binary-searches its own run of the group (with one lane, kSearchGroup runs advance in
// lock-step), so the probes are independent loads in flight together, and the insertion
// positions reach the query's lanes by a DPP quad broadcast.
#include "zeta_internal.hpp"
#include "xlane.hpp"

namespace zeta {

constexpr int kSearchGroup = 2;  // runs whose binary searches advance in lock-step
constexpr int kChunk = 8;        // candidates of a walk loaded per step (register budget)
constexpr int kChunkGroup = 4;   // chunks whose searches advance in lock-step (chunked search)
constexpr int kInsert = 2;       // walk candidates merged by insertion when no more can enter
// The second insertion tier (lane groups of 4 or more lanes): the first three candidates, or
// four for K = 64 on 8 lanes (measured at N = 65536, H = 8: k = 64 selection 0.334 -> 0.326
// ms; four for K = 16 and 32 was slower, 0.126 and 0.168 against 0.119 and 0.165).
template <int K, int L>
constexpr int insert2_of() { return (K / L >= 8 && L == 8) ? 4 : 3; }
// lanes per query of a list of K entries (measured at N = 65536, H = 8: K = 32 on 4 / 8 / 16
// lanes 0.191 / 0.179 / 0.283 ms; K = 64 on 4 / 8 / 16 lanes 0.55 / 0.34 / 0.43 ms)
constexpr int kLanes64 = 8;      // 8 entries per lane
constexpr int kLanes32 = 8;      // 4 entries per lane
constexpr int kLanes16 = 4;      // 4 entries per lane (one lane: 0.151 ms, four: 0.120)

// One word of lane `lane ^ D` (D = 1, 2: a DPP quad permute that the compiler can fold into
// the instruction consuming it; D = 4, 8: a ds_swizzle in bitmask mode, and-mask 31 with
// xor-mask D, inside the 32-lane half of the wavefront).  Every lane of the query's group is
// active where these are used, and its partner is in the same group.
template <int D>
__device__ __forceinline__ uint32_t lane_xor32(uint32_t x) {
    if constexpr (D == 1 || D == 2) {
        constexpr int ctrl = D == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
        return static_cast<uint32_t>(
            __builtin_amdgcn_update_dpp(0, static_cast<int>(x), ctrl, 0xF, 0xF, true));
    } else {
        static_assert(D == 4 || D == 8, "partners within a 16-lane row");
        return static_cast<uint32_t>(
            __builtin_amdgcn_ds_swizzle(static_cast<int>(x), 0x1F | (D << 10)));
    }
}

// Value of the lane `lane ^ D` of the same lane group, 64 bits.
template <int D>
__device__ __forceinline__ uint64_t lane_xor64(uint64_t x) {
    const uint32_t lo = lane_xor32<D>(static_cast<uint32_t>(x));
    const uint32_t hi = lane_xor32<D>(static_cast<uint32_t>(x >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t pack64(uint32_t lo, uint32_t hi) {
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// One word of lane SRC of this lane's aligned group of 8 (ds_swizzle in bit-mask mode:
// source lane = (lane & 0x18) | SRC inside the 32-lane half).
template <int SRC>
__device__ __forceinline__ uint32_t group8_lane32(uint32_t x) {
    static_assert(SRC >= 0 && SRC < 8, "a group has 8 lanes");
    return static_cast<uint32_t>(
        __builtin_amdgcn_ds_swizzle(static_cast<int>(x), 0x18 | (SRC << 5)));
}

// One word of lane SRC of this 16-lane row (DPP row_newbcast).
template <int SRC>
__device__ __forceinline__ uint32_t row_lane32(uint32_t x) {
    static_assert(SRC >= 0 && SRC < 16, "a row has 16 lanes");
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x150 + SRC, 0xF, 0xF, true));
}

// Value of the last lane of this query's lane group (L = 1, 2 or 4 lanes in a quad, or a
// 16-lane row).
template <int L>
__device__ __forceinline__ uint64_t from_last_lane(uint64_t x) {
    static_assert(L == 1 || L == 2 || L == 4 || L == 8 || L == 16,
                  "lane groups of 1, 2, 4, 8 or 16");
    if constexpr (L == 1) {
        return x;
    } else if constexpr (L == 8) {
        return pack64(group8_lane32<7>(static_cast<uint32_t>(x)),
                      group8_lane32<7>(static_cast<uint32_t>(x >> 32)));
    } else if constexpr (L == 16) {
        return pack64(row_lane32<15>(static_cast<uint32_t>(x)),
                      row_lane32<15>(static_cast<uint32_t>(x >> 32)));
    } else {
        constexpr int ctrl = L == 2 ? 0xF5 : 0xFF;  // quad_perm [1,1,3,3] / [3,3,3,3]
        const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(x)), ctrl,
                                                0xF, 0xF, false);
        const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(x >> 32)),
                                                ctrl, 0xF, 0xF, false);
        return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
    }
}

// Value of lane SRC of this query's lane group (L = 1, 2 or 4 lanes in a quad, or a 16-lane
// row), 64 bits.
template <int L, int SRC>
__device__ __forceinline__ uint64_t from_lane64(uint64_t x) {
    if constexpr (L == 1) {
        return x;
    } else if constexpr (L == 8) {
        return pack64(group8_lane32<SRC>(static_cast<uint32_t>(x)),
                      group8_lane32<SRC>(static_cast<uint32_t>(x >> 32)));
    } else if constexpr (L == 16) {
        return pack64(row_lane32<SRC>(static_cast<uint32_t>(x)),
                      row_lane32<SRC>(static_cast<uint32_t>(x >> 32)));
    } else {
        constexpr int ctrl = L == 4 ? SRC * 0x55 : (SRC * 0x5) | ((2 + SRC) * 0x50);
        const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(x)), ctrl,
                                                0xF, 0xF, false);
        const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(x >> 32)),
                                                ctrl, 0xF, 0xF, false);
        return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
    }
}

// Value of lane SRC of this query's lane group (L = 1, 2 or 4 lanes in a quad, or a 16-lane
// row); x < 2^32.
template <int L, int SRC>
__device__ __forceinline__ int64_t from_lane(int64_t x) {
    if constexpr (L == 1) {
        return x;
    } else if constexpr (L == 8) {
        return static_cast<int64_t>(group8_lane32<SRC>(static_cast<uint32_t>(x)));
    } else if constexpr (L == 16) {
        return static_cast<int64_t>(row_lane32<SRC>(static_cast<uint32_t>(x)));
    } else {
        // quad_perm [SRC, SRC, SRC, SRC] for a quad; [SRC, SRC, 2+SRC, 2+SRC] for lane pairs
        constexpr int ctrl = L == 4 ? SRC * 0x55 : (SRC * 0x5) | ((2 + SRC) * 0x50);
        return static_cast<int64_t>(static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(
            static_cast<int>(static_cast<uint32_t>(x)), ctrl, 0xF, 0xF, false)));
    }
}

// Packed keys (|dz| << S) | j.  With 30-bit codes (S = 32) a key is below 2^62, so its bit
// pattern read as an IEEE double is non-negative and finite (subnormal while |dz| < 2^20),
// and for such patterns the double order is the integer order.  A compare-exchange is then
// one v_min_f64 and one v_max_f64 instead of 64-bit compares and two selects per output; the
// kernels keep f64 subnormals (the default FP mode), so no pattern is flushed, and neither
// instruction changes a non-NaN input.  The empty slot is 2^62 - 1, above every key (j <
// 2^31).  With 36-bit codes (S = 28) keys use all 64 bits: integer compares, empty = ~0.
template <int S>
constexpr uint64_t kNone = S == 32 ? 0x3fffffffffffffffull : ~0ull;

template <int S>
__device__ __forceinline__ uint64_t kmin(uint64_t a, uint64_t b) {
    if constexpr (S == 32) {
        uint64_t r;
        asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
        return r;
    } else {
        return b < a ? b : a;
    }
}

template <int S>
__device__ __forceinline__ uint64_t kmax(uint64_t a, uint64_t b) {
    if constexpr (S == 32) {
        uint64_t r;
        asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
        return r;
    } else {
        return b < a ? a : b;
    }
}

// Cross-lane compare-exchange stage with partner lane ^ D: the lower lane keeps minima.
// 30-bit-code keys: a lane that keeps maxima negates both operands (flips the sign bit of the
// high word; the partner's arrives flipped from the DPP instruction that fetches it), takes
// the one v_min_f64 -- the negated maximum -- and flips the result back.
template <int E, int D, int S>
__device__ __forceinline__ void cross_stage(uint64_t (&a)[E], bool keep_min) {
    if constexpr (S == 32) {
        const uint32_t m = keep_min ? 0u : 0x80000000u;
#pragma unroll
        for (int u = 0; u < E; ++u) {
            const uint32_t lo = static_cast<uint32_t>(a[u]), hi = static_cast<uint32_t>(a[u] >> 32);
            const uint64_t y = pack64(lane_xor32<D>(lo), lane_xor32<D>(hi) ^ m);
            const uint64_t r = kmin<S>(pack64(lo, hi ^ m), y);
            a[u] = pack64(static_cast<uint32_t>(r), static_cast<uint32_t>(r >> 32) ^ m);
        }
    } else {
#pragma unroll
        for (int u = 0; u < E; ++u) {
            const uint64_t y = lane_xor64<D>(a[u]);
            const bool lt = y < a[u];
            a[u] = (lt == keep_min) ? y : a[u];
        }
    }
}

// The two cross-lane stages of a clean over a quad (partners lane ^ 2, then lane ^ 1) on
// 30-bit-code keys, chained in signed form: after the first stage a value stays negated by
// its lane's first mask, and the second stage re-signs both operands by the xor of the two
// masks (a lane and its ^ 1 partner share the first mask), so one flip per stage remains.
template <int E>
__device__ __forceinline__ void cross_stages_quad(uint64_t (&a)[E], int lane) {
    const uint32_t m2 = (lane & 2) ? 0x80000000u : 0u;
    const uint32_t m1 = (lane & 1) ? 0x80000000u : 0u;
    const uint32_t m12 = m1 ^ m2;
#pragma unroll
    for (int u = 0; u < E; ++u) {
        uint32_t lo = static_cast<uint32_t>(a[u]), hi = static_cast<uint32_t>(a[u] >> 32);
        const uint64_t r2 = kmin<32>(pack64(lo, hi ^ m2),
                                     pack64(lane_xor32<2>(lo), lane_xor32<2>(hi) ^ m2));
        lo = static_cast<uint32_t>(r2);
        hi = static_cast<uint32_t>(r2 >> 32);  // negated by m2
        const uint64_t r1 = kmin<32>(pack64(lo, hi ^ m12),
                                     pack64(lane_xor32<1>(lo), lane_xor32<1>(hi) ^ m12));
        a[u] = pack64(static_cast<uint32_t>(r1), static_cast<uint32_t>(r1 >> 32) ^ m1);
    }
}

// Sort the bitonic sequence held as L lanes x E registers (lane-major) ascending.
template <int E, int L, int S>
__device__ __forceinline__ void bitonic_clean(uint64_t (&a)[E], int lane) {
    if constexpr (L >= 16) cross_stage<E, 8, S>(a, (lane & 8) == 0);
    if constexpr (L >= 8) cross_stage<E, 4, S>(a, (lane & 4) == 0);
    if constexpr (L >= 4 && S == 32) {
        cross_stages_quad<E>(a, lane);
    } else {
        if constexpr (L >= 4) cross_stage<E, 2, S>(a, (lane & 2) == 0);
        if constexpr (L >= 2) cross_stage<E, 1, S>(a, (lane & 1) == 0);
    }
#pragma unroll
    for (int stride = E / 2; stride > 0; stride >>= 1) {
#pragma unroll
        for (int t = 0; t < E; ++t) {
            if ((t & stride) == 0) {
                const uint64_t x = a[t], y = a[t + stride];
                a[t] = kmin<S>(x, y);
                a[t + stride] = kmax<S>(x, y);
            }
        }
    }
}

// One compare-exchange layer of a bitonic sort of the K = E*L entries (entry x = lane*E + t)
// for block size K2 and stride J; DESC sorts descending.
template <int E, int L, int K2, int J, bool DESC, int S>
__device__ __forceinline__ void sort_layer(uint64_t (&a)[E], int lane) {
    if constexpr (J >= E) {
        const int x = lane * E;
        const bool up = ((x & K2) == 0) != DESC;
        cross_stage<E, J / E, S>(a, up == ((x & J) == 0));
    } else {
#pragma unroll
        for (int t = 0; t < E; ++t) {
            if ((t & J) == 0) {
                const int x = lane * E + t;
                const bool up = ((x & K2) == 0) != DESC;
                const uint64_t p = a[t], q = a[t + J];
                const uint64_t lo = kmin<S>(p, q), hi = kmax<S>(p, q);
                a[t] = up ? lo : hi;
                a[t + J] = up ? hi : lo;
            }
        }
    }
    if constexpr (J > 1) sort_layer<E, L, K2, J / 2, DESC, S>(a, lane);
}

template <int E, int L, int K2, bool DESC, int S>
__device__ __forceinline__ void sort_blocks(uint64_t (&a)[E], int lane) {
    if constexpr (K2 <= E * L) {  // a single entry (K = 1) needs no layer
        sort_layer<E, L, K2, K2 / 2, DESC, S>(a, lane);
        if constexpr (K2 < E * L) sort_blocks<E, L, K2 * 2, DESC, S>(a, lane);
    }
}

// Value of the previous lane of this query's lane group (L = 2 or 4 lanes in a quad, or a
// group of 8 or 16); the group's first lane reads its own (quads) or another lane's value
// (larger groups), which the caller replaces.
template <int L>
__device__ __forceinline__ uint64_t from_prev_lane(uint64_t x) {
    // quad_perm [0,0,1,2] / [0,0,2,2]; row_shr:1 for groups of 8 or 16 (the group's first
    // lane then reads the previous group's last lane, which the caller discards)
    constexpr int ctrl = L >= 8 ? 0x111 : (L == 4 ? 0x90 : 0xA0);
    const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(x)), ctrl, 0xF,
                                            0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(x >> 32)), ctrl,
                                            0xF, 0xF, false);
    return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

// Merge R ascending candidates c_0 <= ... <= c_{R-1}, the same on every lane of the query,
// into the ascending list (L lanes x E registers, lane-major).  Entry t of the merged list is
// the t-th smallest of the union of two sorted lists: the least of b_t and of
// max(b_{t-1-r}, c_r) for r < R, where entries before the list's first count as the smallest
// key, 0.  That is 2R min/max per entry and one lane shift per r, against log2(K)
// compare-exchange stages for a bitonic merge.
template <int E, int L, int R, int S>
__device__ __forceinline__ void insert_few(uint64_t (&best)[E], const uint64_t (&c)[R], int lane) {
    static_assert(R <= E, "the shifted entries come from the previous lane only");
    uint64_t prev[R];  // prev[r]: list entry lane*E - 1 - r
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if constexpr (L == 1) {
            prev[r] = 0;
        } else {
            const uint64_t y = from_prev_lane<L>(best[E - 1 - r]);
            prev[r] = lane == 0 ? 0 : y;
        }
    }
    uint64_t out[E];
#pragma unroll
    for (int t = 0; t < E; ++t) {
        uint64_t v = best[t];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int u = t - 1 - r;
            v = kmin<S>(v, kmax<S>(u >= 0 ? best[u] : prev[-1 - u], c[r]));
        }
        out[t] = v;
    }
#pragma unroll
    for (int t = 0; t < E; ++t) best[t] = out[t];
}

// True when no lane group of L lanes (aligned in the wavefront) has two bits set in m.
template <int L>
__device__ __forceinline__ bool one_per_group(uint64_t m) {
    if constexpr (L == 1) {
        return true;
    } else {
        const uint64_t pair_both = m & (m >> 1) & 0x5555555555555555ull;
        if constexpr (L == 2) {
            return pair_both == 0;
        } else if constexpr (L == 8 || L == 16) {
            bool ok = true;
#pragma unroll
            for (int g = 0; g < 64 / L; ++g) {
                const uint32_t c = static_cast<uint32_t>(m >> (L * g)) & ((1u << L) - 1u);
                ok = ok && (c & (c - 1u)) == 0u;
            }
            return ok;
        } else {
            const uint64_t pair_any = (m | (m >> 1)) & 0x5555555555555555ull;
            return pair_both == 0 && (pair_any & (pair_any >> 2) & 0x1111111111111111ull) == 0;
        }
    }
}

// Merge E*L unsorted candidates (lane-major, empty = kNone) into the running top-K.  Nothing
// is done when no candidate beats its query's K-th anywhere in the wavefront (once the prefix
// is long the recent keys rarely do); when no query has two that do, the one that can enter
// is the query's smallest and is inserted; otherwise the candidates are bitonic-sorted
// (descending) and merged.  Each choice is uniform over the active lanes.
template <int E, int L, int S>
__device__ __forceinline__ void merge_unsorted(uint64_t (&best)[E], uint64_t (&cand)[E], int lane) {
    const uint64_t kth = from_last_lane<L>(best[E - 1]);
    int below = 0;
#pragma unroll
    for (int t = 0; t < E; ++t) below += cand[t] < kth ? 1 : 0;
    const uint64_t any = __ballot(below > 0);
    if (any == 0) return;
    if (__ballot(below > 1) == 0 && one_per_group<L>(any)) {
        uint64_t mn[1] = {cand[0]};
#pragma unroll
        for (int t = 1; t < E; ++t) mn[0] = kmin<S>(mn[0], cand[t]);
        if constexpr (L >= 2) mn[0] = kmin<S>(mn[0], lane_xor64<1>(mn[0]));
        if constexpr (L >= 4) mn[0] = kmin<S>(mn[0], lane_xor64<2>(mn[0]));
        if constexpr (L >= 8) mn[0] = kmin<S>(mn[0], lane_xor64<4>(mn[0]));
        if constexpr (L >= 16) mn[0] = kmin<S>(mn[0], lane_xor64<8>(mn[0]));
        insert_few<E, L, 1, S>(best, mn, lane);
        return;
    }
    sort_blocks<E, L, 2, true, S>(cand, lane);
#pragma unroll
    for (int t = 0; t < E; ++t) best[t] = kmin<S>(cand[t], best[t]);
    bitonic_clean<E, L, S>(best, lane);
}

// Entries of one (b,h)'s tree levels are addressed from the slice base.  When the slice holds
// fewer than 2^28 entries per tree (O32) offsets are 32-bit and a load is a uniform base plus
// a 32-bit byte offset; otherwise 64-bit indices.
template <bool O32>
struct TreeIx;
template <>
struct TreeIx<true> {
    using T = int32_t;
    __device__ __forceinline__ static uint64_t load(const uint64_t* base, int32_t i) {
        return *reinterpret_cast<const uint64_t*>(reinterpret_cast<const char*>(base) +
                                                  static_cast<uint32_t>(i) * 8u);
    }
    // the high word of entry i (little-endian: bytes 8 i + 4 .. 8 i + 7)
    __device__ __forceinline__ static uint32_t load_hi(const uint64_t* base, int32_t i) {
        return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(base) +
                                                  (static_cast<uint32_t>(i) * 8u + 4u));
    }
};
template <>
struct TreeIx<false> {
    using T = int64_t;
    __device__ __forceinline__ static uint64_t load(const uint64_t* base, int64_t i) {
        return base[i];
    }
    __device__ __forceinline__ static uint32_t load_hi(const uint64_t* base, int64_t i) {
        return reinterpret_cast<const uint32_t*>(base + i)[1];
    }
};

// What a lower_bound probe reads of a tree entry.  With 30-bit codes (S = 32) the code is the
// entry's high word, and comparing it with the query's code decides the step exactly as the
// full entry against target = zq << 32 does (a 32-bit load and compare); with 36-bit codes
// the code spans both words and the probe reads the entry.  gap() is target minus the packed
// code of entry p - 1 with its position bits cleared: a lower bound of the left walk's first
// key.
template <int S>
struct Probe {
    using T = uint64_t;
    __device__ __forceinline__ static T target(uint64_t t) { return t; }
    template <bool O32>
    __device__ __forceinline__ static T load(const uint64_t* base, typename TreeIx<O32>::T i) {
        return TreeIx<O32>::load(base, i);
    }
    __device__ __forceinline__ static T of(uint64_t e) { return e; }
    __device__ __forceinline__ static uint64_t gap(uint64_t t, T below) {
        return t - (below & ~((uint64_t(1) << S) - 1));
    }
};
template <>
struct Probe<32> {
    using T = uint32_t;
    __device__ __forceinline__ static T target(uint64_t t) { return static_cast<uint32_t>(t >> 32); }
    template <bool O32>
    __device__ __forceinline__ static T load(const uint64_t* base, typename TreeIx<O32>::T i) {
        return TreeIx<O32>::load_hi(base, i);
    }
    __device__ __forceinline__ static T of(uint64_t e) { return static_cast<uint32_t>(e >> 32); }
    __device__ __forceinline__ static uint64_t gap(uint64_t t, T below) {
        return t - (static_cast<uint64_t>(below) << 32);
    }
};

// Walks.  Candidate c (0 = first) of the right walk sits at run position p + c (asc tree,
// key = e - target), of the left walk at p - 1 - c (desc tree, key = (target | jmask) - e).
// For a merge, lane `lane` of the query pairs its list entries [lane*E, lane*E + E) with
// candidates K-1-t, i.e. entry u of its share is candidate K-1-lane*E-u: the elementwise
// minimum of the ascending list and the reversed candidates leaves a bitonic sequence of the
// K smallest.  A position outside the run reads the walk's first position (always inside the
// run when the walk is not empty) and becomes the empty key, so no load sits behind a branch.
template <int K, int L, bool RIGHT, bool O32>
struct WalkShare {
    using IX = typename TreeIx<O32>::T;
    static constexpr int E = K / L;
    IX b, lim, p0;
    // right: entry u is run[b - u], valid iff u > lim; left: run[b + u], valid iff u >= lim
    __device__ __forceinline__ WalkShare(IX p, IX s, int lane)
        : b(RIGHT ? p + (K - 1 - lane * E) : p - K + lane * E),
          lim(RIGHT ? b - s : -b),
          p0(RIGHT ? (p < s ? p : s - 1) : (p > 0 ? p - 1 : 0)) {}
    __device__ __forceinline__ bool ok(int u) const { return RIGHT ? u > lim : u >= lim; }
    __device__ __forceinline__ IX at(int u) const { return ok(u) ? b + (RIGHT ? -u : u) : p0; }
};

template <int K, int L, bool RIGHT, int S, bool O32, int U0, int CH>
__device__ __forceinline__ void walk_load(uint64_t (&c)[CH], const uint64_t* __restrict__ tree,
                                          typename TreeIx<O32>::T roff,
                                          const WalkShare<K, L, RIGHT, O32>& w) {
#pragma unroll
    for (int v = 0; v < CH; ++v) c[v] = TreeIx<O32>::load(tree, roff + w.at(U0 + v));
}

// Key of the tree entry e loaded for entry u of the lane's share.
template <int K, int L, bool RIGHT, int S, bool O32>
__device__ __forceinline__ uint64_t walk_key(uint64_t e, const WalkShare<K, L, RIGHT, O32>& w,
                                             int u, uint64_t target) {
    const uint64_t top = target | ((S == 32) ? 0xffffffffull : ((uint64_t(1) << S) - 1));
    return w.ok(u) ? (RIGHT ? e - target : top - e) : kNone<S>;
}

template <int K, int L, bool RIGHT, int S, bool O32, int U0, int CH>
__device__ __forceinline__ void walk_keys(uint64_t (&c)[CH], const WalkShare<K, L, RIGHT, O32>& w,
                                          uint64_t target) {
#pragma unroll
    for (int v = 0; v < CH; ++v) c[v] = walk_key<K, L, RIGHT, S, O32>(c[v], w, U0 + v, target);
}

// Merge one walk into the running top-K, its candidates loaded kChunk at a time (register
// budget for K = 64); the caller has checked that its first candidate may enter the list.
// Deep in the prefix a walk admits a few keys at most: when candidate kInsert cannot beat
// its query's K-th for any query of the wavefront, the first kInsert candidates are merged
// by insertion and the bitonic merge is skipped; with four or more lanes per query, failing
// that, the first insert2_of<K, L>() when the candidate after them cannot enter (each choice
// uniform over the wavefront).
// `few` = false skips those checks for walks that nearly always admit more (the walks of a
// query's two largest runs).
template <int K, int L, bool RIGHT, int S, bool O32>
__device__ __forceinline__ void merge_walk(uint64_t (&best)[K / L], const uint64_t* __restrict__ tree,
                                           typename TreeIx<O32>::T roff, typename TreeIx<O32>::T p,
                                           typename TreeIx<O32>::T s, uint64_t target, int lane,
                                           bool few = true) {
    constexpr int E = K / L;
    constexpr int CH = kChunk < E ? kChunk : E;
    constexpr int kInsert2 = insert2_of<K, L>();
    const WalkShare<K, L, RIGHT, O32> w(p, s, lane);
    if constexpr (L >= 4 && kInsert > 0 && kInsert < kInsert2 && kInsert2 < L) {
        if (few) {
            // lane r of the query loads candidate r first (run position p + r, or p - 1 - r on
            // the left); the whole walk is loaded only when candidate kInsert2 may enter
            using IX = typename TreeIx<O32>::T;
            const IX q = RIGHT ? p + lane : p - 1 - lane;
            const bool in = RIGHT ? q < s : q >= 0;
            const uint64_t e = TreeIx<O32>::load(tree, roff + (in ? q : w.p0));
            const uint64_t top = target | ((S == 32) ? 0xffffffffull : ((uint64_t(1) << S) - 1));
            const uint64_t key = in ? (RIGHT ? e - target : top - e) : kNone<S>;
            const uint64_t kth = from_last_lane<L>(best[E - 1]);
            if (__ballot(lane == kInsert && key < kth) == 0) {
                uint64_t g[kInsert];
                static_for<0, kInsert>([&](auto rc) {
                    constexpr int r = decltype(rc)::value;
                    g[r] = from_lane64<L, r>(key);
                });
                insert_few<E, L, kInsert, S>(best, g, lane);
                return;
            }
            // one more candidate from the same loads when candidate kInsert2 cannot enter
            // (the shifted entries must come from the previous lane: kInsert2 <= E)
            if constexpr (kInsert2 <= E) {
                if (__ballot(lane == kInsert2 && key < kth) == 0) {
                    uint64_t g[kInsert2];
                    static_for<0, kInsert2>([&](auto rc) {
                        constexpr int r = decltype(rc)::value;
                        g[r] = from_lane64<L, r>(key);
                    });
                    insert_few<E, L, kInsert2, S>(best, g, lane);
                    return;
                }
            }
        }
    } else if constexpr (CH == E && kInsert > 0 && kInsert < E) {
        uint64_t c[E];
        walk_load<K, L, RIGHT, S, O32, 0, E>(c, tree, roff, w);
        // candidate r (r < E) is entry E-1-r of the query's last lane
        uint64_t f[kInsert + 1];
#pragma unroll
        for (int r = 0; r <= kInsert; ++r)
            f[r] = walk_key<K, L, RIGHT, S, O32>(c[E - 1 - r], w, E - 1 - r, target);
        const bool more = lane == L - 1 && f[kInsert] < best[E - 1];
        if (__ballot(more) == 0) {
            uint64_t g[kInsert];
#pragma unroll
            for (int r = 0; r < kInsert; ++r) g[r] = from_last_lane<L>(f[r]);
            insert_few<E, L, kInsert, S>(best, g, lane);
            return;
        }
        walk_keys<K, L, RIGHT, S, O32, 0, E>(c, w, target);
#pragma unroll
        for (int v = 0; v < E; ++v) best[v] = kmin<S>(c[v], best[v]);
        bitonic_clean<E, L, S>(best, lane);
        return;
    }
    static_for<0, E / CH>([&](auto ic) {
        constexpr int u0 = decltype(ic)::value * CH;
        uint64_t c[CH];
        walk_load<K, L, RIGHT, S, O32, u0, CH>(c, tree, roff, w);
        walk_keys<K, L, RIGHT, S, O32, u0, CH>(c, w, target);
#pragma unroll
        for (int v = 0; v < CH; ++v) best[u0 + v] = kmin<S>(c[v], best[u0 + v]);
        if (CH < E) __builtin_amdgcn_sched_barrier(0);
    });
    bitonic_clean<E, L, S>(best, lane);
}

// The first walk of a query (the right walk of its largest run) goes into the empty list:
// its candidates are already in (|dz|, j) order, so lane `lane` takes candidates
// [lane*E, lane*E + E) in place -- no merge network.
template <int K, int L, bool O32>
__device__ __forceinline__ void fill_load(uint64_t (&c)[K / L], const uint64_t* __restrict__ tree,
                                          typename TreeIx<O32>::T roff, typename TreeIx<O32>::T p,
                                          typename TreeIx<O32>::T s, int lane) {
    constexpr int E = K / L;
    const typename TreeIx<O32>::T b = p + lane * E;  // entry t: run[b + t], valid while b + t < s
#pragma unroll
    for (int t = 0; t < E; ++t) c[t] = TreeIx<O32>::load(tree, roff + (b + t < s ? b + t : s - 1));
}

template <int K, int L, int S, bool O32>
__device__ __forceinline__ void fill_keys(uint64_t (&best)[K / L], const uint64_t (&c)[K / L],
                                          typename TreeIx<O32>::T p, typename TreeIx<O32>::T s,
                                          uint64_t target, int lane) {
    constexpr int E = K / L;
    const typename TreeIx<O32>::T b = p + lane * E;
#pragma unroll
    for (int t = 0; t < E; ++t) best[t] = b + t < s ? c[t] - target : kNone<S>;
}

// CT, S: code type and position bits of the packed tree entries (uint32_t, 32 for 30-bit
// codes; uint64_t, 28 for the 36-bit codes of 12-bit cells).
// Workgroup of the exact selection: 256 threads up to K = 16; one wavefront for longer lists,
// whose queries run for very different times (measured at N = 65536, H = 8: k = 32 / 64 / 128
// in 0.180 / 0.345 / 0.820 ms with 256 threads, 0.176 / 0.335 / 0.771 ms with 64; k = 16 is
// 0.120 ms either way).
template <int K>
constexpr int sel_threads() { return K <= 16 ? 256 : 64; }

template <int K, int L, typename CT, int S, bool O32>
__global__ void __launch_bounds__(sel_threads<K>()) zeta_select_kernel(const CT* __restrict__ zq,
                                                           const CT* __restrict__ zk,
                                                           const uint64_t* __restrict__ tree_asc,
                                                           const uint64_t* __restrict__ tree_desc,
                                                           const uint32_t* __restrict__ order,
                                                           int64_t N, int stored, int base,
                                                           int topk, int causal, int64_t tph,
                                                           int64_t tiles,
                                                           int64_t per_xcd,
                                                           int32_t* __restrict__ idx) {
    using IX = typename TreeIx<O32>::T;
    constexpr int E = K / L;
    const int64_t tile = xcd_tile(blockIdx.x, per_xcd);
    if (tile >= tiles) return;
    const int64_t bh = tile / tph;  // uniform: tiles never straddle two (b,h)
    constexpr int QPT = sel_threads<K>() / L;  // queries per workgroup
    const int64_t t = (tile - bh * tph) * QPT + threadIdx.x / L;  // processing position
    const int lane = static_cast<int>(threadIdx.x % L);
    if (t >= N) return;  // uniform over the L lanes of a query
    // queries close on the curve search the same parts of the tree, so taking them in the
    // Z-order processing order keeps the probed lines in L2
    const int64_t i = order ? static_cast<int64_t>(order[bh * N + t]) : t;
    const int64_t row = bh * N + i;
    constexpr uint64_t kJMask = (S == 32) ? 0xffffffffull : ((uint64_t(1) << S) - 1);
    const uint64_t target = static_cast<uint64_t>(zq[row]) << S;
    // the trees hold levels base .. base + stored - 1 of every (b,h), level l at (l - base) N
    const uint64_t* hA = tree_asc + bh * stored * N;
    const uint64_t* hD = tree_desc + bh * stored * N;

    uint64_t best[E];
#pragma unroll
    for (int t = 0; t < E; ++t) best[t] = kNone<S>;

    // The runs are the set bits of the number of usable keys (i+1 under the causal mask,
    // else N), largest first, taken kSearchGroup at a time: their lower_bound searches
    // (first entry with code >= zq) advance together.  Runs shorter than 2K together are the
    // last (m mod 2K) positions, read straight from the codes below.
    const uint64_t m = causal ? static_cast<uint64_t>(i) + 1 : static_cast<uint64_t>(N);
    constexpr uint64_t kShort = 2 * K;
    uint64_t rem = m & ~(kShort - 1);
    // Runs above the top stored level (only m = 2^(top+1) = N under the causal mask, when
    // that level is not built) are taken as runs of the top level; `start` is the first
    // position of the next run, the sum of the runs taken before it.
    const int top = base + stored - 1;
    uint64_t start = 0;
    // A group takes the next kRuns runs (largest first).  With several lanes per query each
    // lane binary-searches its own run(s) of the group (kPer per lane, in lock-step), and the
    // insertion positions then reach every lane of the query by a DPP quad broadcast.
    constexpr int kPer = L == 1 ? kSearchGroup : 1;
    constexpr int kRuns = kPer * L;
    bool fresh = true;  // the list is still empty
    while (rem) {
        // run gi: level l, entries hA[roff .. roff + 2^l) (same in hD); offsets (not
        // pointers) keep every access a global-memory access.  Every lane peels the same
        // runs off `rem` but keeps only its own (gi = lane * kPer + t, level mlv[t] or -1,
        // offset mro[t]); the merges below fetch a run's level and offset from its lane, so
        // no lane holds all of them.
        int lv0 = -1;  // the group's first (largest) run, on every lane
        int mlv[kPer];
        IX mro[kPer];
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            mlv[t] = -1;
            mro[t] = 0;
        }
#pragma unroll
        for (int gi = 0; gi < kRuns; ++gi) {
            if (rem) {
                const int hb = 63 - __clzll(rem);
                const int l = hb < top ? hb : top;
                rem -= uint64_t(1) << l;
                const IX ro = static_cast<IX>(static_cast<int64_t>(l - base) * N +
                                              static_cast<int64_t>(start));
                start += uint64_t(1) << l;
                if (gi == 0) lv0 = l;
                if (lane == gi / kPer) {
                    mlv[gi % kPer] = l;
                    mro[gi % kPer] = ro;
                }
            }
        }
        IX mlen[kPer], pos[kPer];
        bool mon[kPer];
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            mon[t] = mlv[t] >= 0;
            mlen[t] = mlv[t] >= 0 ? IX(1) << mlv[t] : 1;
            pos[t] = 0;
        }
        // probes from clamped positions, held live together (see keep()), so the searches'
        // loads are in flight together.  A lower_bound search by halving steps probes both
        // neighbours of the insertion position p: the probe of the last step that moved is
        // entry p - 1 and the final probe, when it does not move, is entry p.  They give the
        // right walk's first key exactly and a lower bound of the left walk's first key
        // (same code as entry p - 1), so a walk is skipped without loading anything.
        // With 30-bit codes a probe compares codes only, so it reads the entry's high word.
        using PV = typename Probe<S>::T;
        const PV ptarget = Probe<S>::target(target);
        PV below[kPer];
        uint64_t rfirst[kPer], lbound[kPer];
#pragma unroll
        for (int t = 0; t < kPer; ++t) below[t] = 0;
        for (IX step = (IX(1) << lv0) >> 1; step > 0; step >>= 1) {
            PV e[kPer];
#pragma unroll
            for (int t = 0; t < kPer; ++t) {
                const IX at = pos[t] + step - 1;
                e[t] = Probe<S>::template load<O32>(hA, mro[t] + (at < mlen[t] ? at : mlen[t] - 1));
            }
#pragma unroll
            for (int t = 0; t < kPer; ++t) keep(e[t]);
#pragma unroll
            for (int t = 0; t < kPer; ++t) {
                if (pos[t] + step < mlen[t] && e[t] < ptarget) {
                    pos[t] += step;
                    below[t] = e[t];
                }
            }
        }
        {
            uint64_t e[kPer];
#pragma unroll
            for (int t = 0; t < kPer; ++t) e[t] = TreeIx<O32>::load(hA, mro[t] + pos[t]);
#pragma unroll
            for (int t = 0; t < kPer; ++t) keep(e[t]);
#pragma unroll
            for (int t = 0; t < kPer; ++t) {
                // a move here means every entry of the run is below the target
                const bool mv = mon[t] && e[t] < target;
                if (mv) {
                    pos[t] += 1;
                    below[t] = Probe<S>::of(e[t]);
                }
                rfirst[t] = mv || !mon[t] ? kNone<S> : e[t] - target;
                lbound[t] = pos[t] == 0 ? kNone<S> : Probe<S>::gap(target, below[t]);
            }
        }
        static_for<0, kRuns>([&](auto gc) {
            constexpr int gi = decltype(gc)::value;
            constexpr int src = gi / kPer, slot = gi % kPer;
            const IX pg = static_cast<IX>(from_lane<L, src>(pos[slot]));
            const uint64_t rf = from_lane64<L, src>(rfirst[slot]);
            const uint64_t lb = from_lane64<L, src>(lbound[slot]);
            // the run's level and offset, from the lane that searched it
            const int lvg = static_cast<int>(static_cast<uint32_t>(
                from_lane<L, src>(static_cast<uint32_t>(mlv[slot]))));
            IX rog;
            if constexpr (O32)
                rog = static_cast<IX>(from_lane<L, src>(static_cast<uint32_t>(mro[slot])));
            else
                rog = static_cast<IX>(from_lane64<L, src>(static_cast<uint64_t>(mro[slot])));
            if (lvg >= 0) {
                const IX s = IX(1) << lvg;
                const bool fill = gi == 0 && fresh;  // uniform: every query's first group
                if (fill) {
                    uint64_t c[E];
                    fill_load<K, L, O32>(c, hA, rog, pg, s, lane);
#pragma unroll
                    for (int t = 0; t < E; ++t) keep(c[t]);
                    fill_keys<K, L, S, O32>(best, c, pg, s, target, lane);
                } else if (rf < from_last_lane<L>(best[E - 1])) {
                    merge_walk<K, L, true, S, O32>(best, hA, rog, pg, s, target, lane,
                                                   !(fresh && gi < 2));
                }
                if (lb < from_last_lane<L>(best[E - 1]))
                    merge_walk<K, L, false, S, O32>(best, hD, rog, pg, s, target, lane,
                                                    !(fresh && gi < 2));
            }
        });
        fresh = false;
    }

    // the short runs: positions [m - (m mod 2K), m), at most 2K - 1 keys in two groups of K,
    // each merged as unsorted candidates
    {
        const uint64_t z = static_cast<uint64_t>(zq[row]);
        const int64_t sbase = static_cast<int64_t>(m & ~(kShort - 1));
        const int scount = static_cast<int>(m & (kShort - 1));
        const CT* zkh = zk + bh * N;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int cg = scount - g * K;  // entries of this group (uniform over the lanes)
            if (cg <= 0) break;
            // codes from clamped positions, all loaded before any is used
            CT code[E];
#pragma unroll
            for (int t = 0; t < E; ++t) {
                const int u = lane * E + t;
                code[t] = zkh[sbase + g * K + (u < cg ? u : cg - 1)];
            }
#pragma unroll
            for (int t = 0; t < E; ++t) keep(code[t]);
            uint64_t cand[E];
#pragma unroll
            for (int t = 0; t < E; ++t) {
                const int u = lane * E + t;
                cand[t] = kNone<S>;
                if (u < cg) {
                    const int64_t j = sbase + g * K + u;
                    const uint64_t c = static_cast<uint64_t>(code[t]);
                    const uint64_t dz = c > z ? c - z : z - c;
                    cand[t] = (dz << S) | static_cast<uint64_t>(j);
                }
            }
            merge_unsorted<E, L, S>(best, cand, lane);
        }
    }

    int32_t* out = idx + row * topk + lane * E;
#pragma unroll
    for (int t = 0; t < E; ++t)
        if (lane * E + t < topk)
            out[t] = best[t] == kNone<S> ? -1 : static_cast<int32_t>(best[t] & kJMask);
}

template <int K, int L, typename CT, int S>
static hipError_t launch_select_k(int64_t rows, int64_t N, int stored, int base, int topk,
                                  int causal,
                                  const CT* zq, const CT* zk, const uint64_t* ta,
                                  const uint64_t* td, const uint32_t* order, int32_t* idx,
                                  hipStream_t s) {
    // tiles of sel_threads<K>() / L queries, never straddling two (b,h)
    constexpr int QPT = sel_threads<K>() / L;
    const int64_t tph = (N + QPT - 1) / QPT;
    const int64_t tiles = (rows / N) * tph;
    const int64_t per = xcd_per(tiles);
    const dim3 grid(static_cast<unsigned>(per * kXcds));
    if (static_cast<int64_t>(stored) * N < (int64_t(1) << 28))
        hipLaunchKernelGGL((zeta_select_kernel<K, L, CT, S, true>), grid, dim3(sel_threads<K>()), 0, s, zq, zk,
                           ta, td, order, N, stored, base, topk, causal, tph, tiles, per, idx);
    else
        hipLaunchKernelGGL((zeta_select_kernel<K, L, CT, S, false>), grid, dim3(sel_threads<K>()), 0, s, zq,
                           zk, ta, td, order, N, stored, base, topk, causal, tph, tiles, per, idx);
    return hipGetLastError();
}

template <typename CT, int S>
static hipError_t select_t(int64_t BH, int64_t N, int stored, int base, int topk, bool causal,
                           const CT* zq, const CT* zk, const uint64_t* ta, const uint64_t* td,
                           const uint32_t* order, int32_t* idx, hipStream_t s) {
    const int64_t rows = BH * N;
    if (rows <= 0) return hipSuccess;
    // Every run the kernel takes lies on a stored level: the stored levels must reach from
    // log2(2K) (shorter runs are read from the codes) up; runs longer than the top stored
    // level are taken as several runs of that level.
    const int first = select_first_level(topk);
    if ((int64_t(1) << first) <= N && (base > first || base + stored - 1 < first))
        return hipErrorInvalidValue;
    const int c = causal ? 1 : 0;
    if (topk <= 1) return launch_select_k<1, 1, CT, S>(rows, N, stored, base, topk, c, zq, zk, ta, td, order, idx, s);
    if (topk <= 2) return launch_select_k<2, 1, CT, S>(rows, N, stored, base, topk, c, zq, zk, ta, td, order, idx, s);
    if (topk <= 4) return launch_select_k<4, 1, CT, S>(rows, N, stored, base, topk, c, zq, zk, ta, td, order, idx, s);
    if (topk <= 8) return launch_select_k<8, 1, CT, S>(rows, N, stored, base, topk, c, zq, zk, ta, td, order, idx, s);
    if (topk <= 16) return launch_select_k<16, kLanes16, CT, S>(rows, N, stored, base, topk, c, zq, zk, ta, td, order, idx, s);
    if (topk <= 32) return launch_select_k<32, kLanes32, CT, S>(rows, N, stored, base, topk, c, zq, zk, ta, td, order, idx, s);
    if (topk <= 64) return launch_select_k<64, kLanes64, CT, S>(rows, N, stored, base, topk, c, zq, zk, ta, td, order, idx, s);
    if (topk <= 128) return launch_select_k<128, 16, CT, S>(rows, N, stored, base, topk, c, zq, zk, ta, td, order, idx, s);
    return launch_select_k<256, 16, CT, S>(rows, N, stored, base, topk, c, zq, zk, ta, td, order, idx, s);
}

hipError_t launch_select(int64_t BH, int64_t N, int stored, int base, int topk, bool causal,
                         const uint32_t* zq, const uint32_t* zk, const uint64_t* tree_asc,
                         const uint64_t* tree_desc, const uint32_t* order, int32_t* idx,
                         hipStream_t s) {
    return select_t<uint32_t, 32>(BH, N, stored, base, topk, causal, zq, zk, tree_asc, tree_desc,
                                  order, idx, s);
}

hipError_t launch_select36(int64_t BH, int64_t N, int stored, int base, int topk, bool causal,
                           const uint64_t* zq, const uint64_t* zk, const uint64_t* tree_asc,
                           const uint64_t* tree_desc, const uint32_t* order, int32_t* idx,
                           hipStream_t s) {
    return select_t<uint64_t, 28>(BH, N, stored, base, topk, causal, zq, zk, tree_asc, tree_desc,
                                  order, idx, s);
}

int select_first_level(int topk) {
    int k = 1;
    while (k < topk) k <<= 1;  // K: topk padded to a power of two
    int l = 0;
    while ((1 << l) < 2 * k) ++l;
    return l;  // log2(2K): shorter runs are read from the codes
}

// ---------------------------------------------------------------------------- chunked
// The pages' chunked causal search (summary page, "Approach": keys sorted and chunked so all
// queries search in parallel under the causal mask; rebuttal page, answer W2/A2: 4 to 32
// chunks, and the window centred at the query's insertion position in the sorted keys).
// Chunks are the aligned blocks of 2^lvl positions, i.e. one level of the merge-sort tree
// (ascending (code, j)).  For every chunk up to the query's own: lower_bound p of zq, the
// window of min(k, n) sorted entries from p - floor(k/2) shifted inside the chunk, keys
// j > i dropped.  A window is in (code, j) order, which is not (|dz|, j) order inside a
// group of equal codes below zq, so its candidates are bitonic-sorted (descending) across
// the query's lanes and then merged into the running top-K like a walk (the windows of
// most chunks admit keys, so the skip and insertion checks of the exact search only cost
// here).

template <int K, int L, typename CT, int S>
__global__ void __launch_bounds__(256) zeta_select_chunked_kernel(
    const CT* __restrict__ zq, const uint64_t* __restrict__ tree_asc, int64_t rows,
    int64_t N, int stored, int base, int lvl, int topk, int32_t* __restrict__ idx) {
    constexpr int E = K / L;
    constexpr uint64_t kJMask = (S == 32) ? 0xffffffffull : ((uint64_t(1) << S) - 1);
    const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t row = g / L;
    const int lane = static_cast<int>(g % L);
    if (row >= rows) return;  // uniform over the L lanes of a query
    const int64_t bh = row / N;
    const int64_t i = row - bh * N;
    const uint64_t z = zq[row];
    const uint64_t target = z << S;
    const uint64_t* run = tree_asc + bh * stored * N + static_cast<int64_t>(lvl - base) * N;
    const int64_t len = int64_t(1) << lvl;

    uint64_t best[E];
#pragma unroll
    for (int t = 0; t < E; ++t) best[t] = kNone<S>;

    // chunks 0 .. i >> lvl, kChunkGroup at a time: their lower_bound searches advance in
    // lock-step (probes from clamped positions, in flight together), then each chunk's window
    // is loaded in one batch and merged
    const int64_t nch = (i >> lvl) + 1;
    for (int64_t c0 = 0; c0 < nch; c0 += kChunkGroup) {
        int64_t lo[kChunkGroup], n[kChunkGroup], p[kChunkGroup];
#pragma unroll
        for (int gi = 0; gi < kChunkGroup; ++gi) {
            const int64_t c = c0 + gi < nch ? c0 + gi : nch - 1;
            lo[gi] = c * len;
            n[gi] = N - lo[gi] < len ? N - lo[gi] : len;
            p[gi] = 0;
        }
        for (int64_t step = len >> 1; step > 0; step >>= 1) {
            uint64_t e[kChunkGroup];
#pragma unroll
            for (int gi = 0; gi < kChunkGroup; ++gi) {
                const int64_t at = p[gi] + step - 1;
                e[gi] = run[lo[gi] + (at < n[gi] ? at : n[gi] - 1)];
            }
#pragma unroll
            for (int gi = 0; gi < kChunkGroup; ++gi) keep(e[gi]);
#pragma unroll
            for (int gi = 0; gi < kChunkGroup; ++gi)
                if (p[gi] + step <= n[gi] && e[gi] < target) p[gi] += step;
        }
        {
            uint64_t e[kChunkGroup];
#pragma unroll
            for (int gi = 0; gi < kChunkGroup; ++gi)
                e[gi] = run[lo[gi] + (p[gi] < n[gi] ? p[gi] : n[gi] - 1)];
#pragma unroll
            for (int gi = 0; gi < kChunkGroup; ++gi) keep(e[gi]);
#pragma unroll
            for (int gi = 0; gi < kChunkGroup; ++gi)
                if (p[gi] < n[gi] && e[gi] < target) p[gi] += 1;
        }
#pragma unroll
        for (int gi = 0; gi < kChunkGroup; ++gi) {
            if (c0 + gi >= nch) break;  // uniform over the query's lanes
            const int64_t w = topk < n[gi] ? topk : n[gi];  // window of k entries (K pads k)
            int64_t w0 = p[gi] - topk / 2;
            if (w0 > n[gi] - w) w0 = n[gi] - w;
            if (w0 < 0) w0 = 0;
            uint64_t ev[E];
#pragma unroll
            for (int t = 0; t < E; ++t) {
                const int64_t u = lane * E + t;
                ev[t] = run[lo[gi] + w0 + (u < w ? u : w - 1)];
            }
#pragma unroll
            for (int t = 0; t < E; ++t) keep(ev[t]);
            uint64_t cand[E];
#pragma unroll
            for (int t = 0; t < E; ++t) {
                const int64_t u = lane * E + t;
                cand[t] = kNone<S>;
                if (u < w) {
                    const uint64_t j = ev[t] & kJMask;
                    const uint64_t code = ev[t] >> S;
                    const uint64_t dz = code > z ? code - z : z - code;
                    if (static_cast<int64_t>(j) <= i) cand[t] = (dz << S) | j;  // causal mask
                }
            }
            sort_blocks<E, L, 2, true, S>(cand, lane);
#pragma unroll
            for (int t = 0; t < E; ++t) best[t] = kmin<S>(cand[t], best[t]);
            bitonic_clean<E, L, S>(best, lane);
        }
    }

    int32_t* out = idx + row * topk + lane * E;
#pragma unroll
    for (int t = 0; t < E; ++t)
        if (lane * E + t < topk)
            out[t] = best[t] == kNone<S> ? -1 : static_cast<int32_t>(best[t] & kJMask);
}

template <int K, int L, typename CT, int S>
static hipError_t launch_chunked_k(int64_t rows, int64_t N, int stored, int base, int lvl,
                                   int topk,
                                   const CT* zq, const uint64_t* ta, int32_t* idx,
                                   hipStream_t s) {
    const int64_t blocks = (rows * L + 255) / 256;
    hipLaunchKernelGGL((zeta_select_chunked_kernel<K, L, CT, S>), dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, s, zq, ta, rows, N, stored, base, lvl, topk, idx);
    return hipGetLastError();
}

template <typename CT, int S>
static hipError_t chunked_t(int64_t BH, int64_t N, int stored, int base, int lvl, int topk,
                            const CT* zq,
                            const uint64_t* ta, int32_t* idx, hipStream_t s) {
    const int64_t rows = BH * N;
    if (rows <= 0) return hipSuccess;
    if (topk <= 1) return launch_chunked_k<1, 1, CT, S>(rows, N, stored, base, lvl, topk, zq, ta, idx, s);
    if (topk <= 2) return launch_chunked_k<2, 1, CT, S>(rows, N, stored, base, lvl, topk, zq, ta, idx, s);
    if (topk <= 4) return launch_chunked_k<4, 1, CT, S>(rows, N, stored, base, lvl, topk, zq, ta, idx, s);
    if (topk <= 8) return launch_chunked_k<8, 1, CT, S>(rows, N, stored, base, lvl, topk, zq, ta, idx, s);
    // lanes per query measured at N = 65536, H = 8: K = 16 on 4 lanes 0.155 ms (C = 4) against
    // 0.170 on one; K = 32 on 2 lanes 0.215 ms against 0.243 on 8
    if (topk <= 16) return launch_chunked_k<16, 4, CT, S>(rows, N, stored, base, lvl, topk, zq, ta, idx, s);
    if (topk <= 32) return launch_chunked_k<32, 2, CT, S>(rows, N, stored, base, lvl, topk, zq, ta, idx, s);
    if (topk <= 64) return launch_chunked_k<64, kLanes64, CT, S>(rows, N, stored, base, lvl, topk, zq, ta, idx, s);
    if (topk <= 128) return launch_chunked_k<128, 16, CT, S>(rows, N, stored, base, lvl, topk, zq, ta, idx, s);
    return launch_chunked_k<256, 16, CT, S>(rows, N, stored, base, lvl, topk, zq, ta, idx, s);
}

hipError_t launch_select_chunked(int64_t BH, int64_t N, int stored, int base, int lvl, int topk,
                                 const uint32_t* zq, const uint64_t* ta, int32_t* idx,
                                 hipStream_t s) {
    return chunked_t<uint32_t, 32>(BH, N, stored, base, lvl, topk, zq, ta, idx, s);
}

hipError_t launch_select_chunked36(int64_t BH, int64_t N, int stored, int base, int lvl,
                                   int topk,
                                   const uint64_t* zq, const uint64_t* ta, int32_t* idx,
                                   hipStream_t s) {
    return chunked_t<uint64_t, 28>(BH, N, stored, base, lvl, topk, zq, ta, idx, s);
}

// ---------------------------------------------------------------------------- curves
// Several curves (rebuttal page, on the asymmetry of interleaving: 3 or 6 coordinate orders,
// each collecting k // P tokens).  sel[c] holds curve c's exact top-per; the result lists
// curve 0's picks, then each later curve's picks not listed yet, in curve order, and -1 in
// the remaining slots.  One thread per query; a pick is a repeat when an earlier curve
// picked it (a curve's own picks are distinct).
__global__ void __launch_bounds__(256) zeta_curves_merge_kernel(const int32_t* __restrict__ sel,
                                                                 int64_t rows, int curves, int per,
                                                                 int topk,
                                                                 int32_t* __restrict__ idx) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (row >= rows) return;
    int32_t* out = idx + row * topk;
    int pos = 0;
    for (int c = 0; c < curves; ++c) {
        const int32_t* mine = sel + (static_cast<int64_t>(c) * rows + row) * per;
        for (int r = 0; r < per; ++r) {
            const int32_t j = mine[r];
            if (j < 0) continue;
            bool seen = false;
            for (int c2 = 0; c2 < c && !seen; ++c2) {
                const int32_t* other = sel + (static_cast<int64_t>(c2) * rows + row) * per;
                for (int r2 = 0; r2 < per; ++r2) seen = seen || other[r2] == j;
            }
            if (!seen) out[pos++] = j;
        }
    }
    for (; pos < topk; ++pos) out[pos] = -1;
}

hipError_t launch_curves_merge(int64_t rows, int curves, int per, int topk, const int32_t* sel,
                               int32_t* idx, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(zeta_curves_merge_kernel, dim3(static_cast<unsigned>((rows + 255) / 256)),
                       dim3(256), 0, s, sel, rows, curves, per, topk, idx);
    return hipGetLastError();
}

}  // namespace zeta
