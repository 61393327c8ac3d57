// tree.hip -- per-(b,h) merge-sort tree of the key codes.
//
// "ZETA: Leveraging Z-order Curves for Efficient Top-k Attention", rebuttal page, answers
// W3/A3 and W2/A2 ("Clarification"): keys are sorted along the Z-order line so that a
// query finds its neighbours by binary search around its insertion position.  Under the
// causal mask a query i may only see keys j <= i, so instead of one sort the keys are kept
// sorted per aligned power-of-two block of positions: level l holds every block
// [m 2^l, (m+1) 2^l) sorted (the last block possibly shorter).  Any prefix [0, i] is the
// union of at most log2(N)+1 such blocks.
//
// Two trees are built from the same codes with different packed keys, both sorted as plain
// ascending uint64 (S = 32 for 30-bit codes; S = 28 for the 36-bit codes of 12-bit cells,
// which holds positions below 2^28):
//   asc : (code << S) | j           -> code ascending, j ascending
//   desc: (code << S) | (~j mod 2^S) -> code ascending, j descending
// The selection kernel walks the asc tree forward (codes >= the query) and the desc tree
// backward (codes < the query), so both walks meet equal codes in ascending j order.
//
// Levels below `first` are not written (the selection reads short runs straight from the
// codes); they are still formed in LDS on the way up.  Only the levels from
// tree_store_base(levels, first) up are stored: level l of (b,h) sits at
// tree + (bh * stored + l - base) * N, stored = levels - base.
// Build: levels 0..10 inside one workgroup per 1024-entry tile (LDS rank merge: each entry
// moves to its own index plus its rank in the sibling block; keys are unique, so this is
// an exact merge), then one merge-path launch per higher level (streaming: 8 B read and
// 8 B written per entry and tree).
#include "zeta_internal.hpp"

namespace zeta {

constexpr int kTileLog = 10;
constexpr int kTile = 1 << kTileLog;
constexpr int kMergeThreads = 256;
constexpr int kMergeTile = 2048;  // merged outputs per workgroup
constexpr int kMergePer = kMergeTile / kMergeThreads;
static_assert(kMergeThreads == 256, "the split search runs two diagonals on 128 threads each");

__device__ __forceinline__ int lds_lower_bound(const uint64_t* a, int n, uint64_t x) {
    int lo = 0;
    while (n > 0) {
        int half = n >> 1;
        if (a[lo + half] < x) {
            lo += half + 1;
            n -= half + 1;
        } else {
            n = half;
        }
    }
    return lo;
}

template <typename CT, int S>
__global__ void __launch_bounds__(kTile) zeta_tree_tile_kernel(const CT* __restrict__ zk,
                                                              uint64_t* __restrict__ asc,
                                                              uint64_t* __restrict__ desc,
                                                              int64_t N, int stored, int top,
                                                              int first) {
    constexpr uint64_t kJMask = (S == 32) ? 0xffffffffull : ((uint64_t(1) << S) - 1);
    __shared__ uint64_t buf[2][2][kTile];  // [tree][ping-pong][entry]
    const int64_t bh = blockIdx.y;
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kTile;
    const int n = static_cast<int>(N - base < kTile ? N - base : kTile);
    const CT* zrow = zk + bh * N + base;
    // level l at (l - first) N: `first` is also the lowest stored level
    uint64_t* tA = asc + bh * stored * N + base;
    uint64_t* tD = desc + bh * stored * N + base;

    for (int e = threadIdx.x; e < n; e += blockDim.x) {
        const uint64_t j = static_cast<uint64_t>(base + e);
        const uint64_t c = static_cast<uint64_t>(zrow[e]) << S;
        const uint64_t ka = c | j, kd = c | (~j & kJMask);
        buf[0][0][e] = ka;
        buf[1][0][e] = kd;
        if (first == 0) {
            tA[e] = ka;
            tD[e] = kd;
        }
    }
    __syncthreads();

    int cur = 0;
    for (int l = 0; l < top; ++l) {
        const int s = 1 << l;
        for (int e = threadIdx.x; e < n; e += blockDim.x) {
            const int run0 = e & ~(2 * s - 1);
            const bool inB = (e & s) != 0;
            const int own = e - run0 - (inB ? s : 0);
            const int sib0 = inB ? run0 : run0 + s;
            int sibLen = n - sib0;
            sibLen = sibLen < 0 ? 0 : (sibLen > s ? s : sibLen);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint64_t x = buf[t][cur][e];
                const int r = lds_lower_bound(&buf[t][cur][sib0], sibLen, x);
                buf[t][cur ^ 1][run0 + own + r] = x;
            }
        }
        __syncthreads();
        cur ^= 1;
        if (l + 1 < first) continue;  // level not read by the caller: stays in LDS only
        uint64_t* oA = tA + static_cast<int64_t>(l + 1 - first) * N;
        uint64_t* oD = tD + static_cast<int64_t>(l + 1 - first) * N;
        for (int e = threadIdx.x; e < n; e += blockDim.x) {
            oA[e] = buf[0][cur][e];
            oD[e] = buf[1][cur][e];
        }
    }
}

// Number of A entries among the first d outputs of merge(A, B) (keys unique).
__device__ __forceinline__ int diag_split(const uint64_t* A, int na, const uint64_t* B, int nb,
                                          int d) {
    int lo = d - nb > 0 ? d - nb : 0;
    int hi = d < na ? d : na;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (A[mid] < B[d - 1 - mid])
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

// Level l -> l+1 for l >= kTileLog: merge sibling blocks of 2^l entries (merge path).
__global__ void __launch_bounds__(kMergeThreads) zeta_tree_merge_kernel(uint64_t* __restrict__ asc,
                                                               uint64_t* __restrict__ desc,
                                                               int64_t N, int stored, int base,
                                                               int l) {
    __shared__ uint64_t seg[kMergeTile];
    __shared__ int split[2];
    const int64_t bh = blockIdx.y;
    uint64_t* T = (blockIdx.z ? desc : asc) + bh * stored * N;
    const uint64_t* src = T + static_cast<int64_t>(l - base) * N;
    uint64_t* dst = T + static_cast<int64_t>(l + 1 - base) * N;
    const int64_t s = int64_t(1) << l;
    const int64_t o0 = static_cast<int64_t>(blockIdx.x) * kMergeTile;
    if (o0 >= N) return;
    const int64_t run0 = o0 & ~(2 * s - 1);
    const int na = static_cast<int>(N - run0 < s ? N - run0 : s);
    int64_t nbl = N - run0 - s;
    const int nb = static_cast<int>(nbl < 0 ? 0 : (nbl > s ? s : nbl));
    const uint64_t* A = src + run0;
    const uint64_t* B = src + run0 + s;
    const int d0 = static_cast<int>(o0 - run0);
    const int d1 = d0 + kMergeTile < na + nb ? d0 + kMergeTile : na + nb;

    // Merge-path splits of the two diagonals d0, d1 (threads 0-127 and 128-255): the number
    // a of A entries among the first d outputs is the first a with A[a] > B[d-1-a] (keys are
    // unique).  Each round tests 128 evenly spaced candidates of the open interval at once,
    // so a few rounds of independent loads replace a long chain of dependent ones.
    {
        __shared__ int lo_s[2], hi_s[2], lo_n[2], hi_n[2];
        const int h = threadIdx.x >> 7;
        const int t = threadIdx.x & 127;
        const int d = h ? d1 : d0;
        if (t == 0) {
            lo_s[h] = d - nb > 0 ? d - nb : 0;
            hi_s[h] = d < na ? d : na;
        }
        __syncthreads();
        while (true) {
            const int lo = lo_s[h], hi = hi_s[h];
            const bool open0 = lo_s[0] < hi_s[0], open1 = lo_s[1] < hi_s[1];
            if (!open0 && !open1) break;  // uniform over the workgroup
            __syncthreads();
            if (t == 0) {
                lo_n[h] = lo;
                hi_n[h] = hi;
            }
            __syncthreads();
            if (lo < hi) {
                const int step = (hi - lo + 127) / 128;
                const int a = lo + t * step;
                if (a < hi) {
                    if (A[a] < B[d - 1 - a])
                        atomicMax(&lo_n[h], a + 1);  // the split lies above a
                    else
                        atomicMin(&hi_n[h], a);      // the split is at most a
                }
            }
            __syncthreads();
            if (t == 0) {
                lo_s[h] = lo_n[h];
                hi_s[h] = hi_n[h];
            }
            __syncthreads();
        }
        if (t == 0) split[h] = lo_s[h];
    }
    __syncthreads();
    const int a0 = split[0], a1 = split[1];
    const int b0 = d0 - a0, b1 = d1 - a1;
    const int ca = a1 - a0, cb = b1 - b0;
    for (int e = threadIdx.x; e < ca + cb; e += blockDim.x)
        seg[e] = e < ca ? A[a0 + e] : B[b0 + e - ca];
    __syncthreads();

    // each thread merges kMergePer consecutive outputs into LDS; the tile is then written out
    // with consecutive lanes on consecutive entries
    __shared__ uint64_t merged[kMergeTile];
    const uint64_t* sa = seg;
    const uint64_t* sb = seg + ca;
    const int t0 = threadIdx.x * kMergePer;
    if (t0 < ca + cb) {
        int ia = diag_split(sa, ca, sb, cb, t0);
        int ib = t0 - ia;
        const int cnt = ca + cb - t0 < kMergePer ? ca + cb - t0 : kMergePer;
        for (int u = 0; u < cnt; ++u) {
            uint64_t x;
            if (ib >= cb || (ia < ca && sa[ia] < sb[ib]))
                x = sa[ia++];
            else
                x = sb[ib++];
            merged[t0 + u] = x;
        }
    }
    __syncthreads();
    uint64_t* out = dst + run0 + d0;
    for (int e = threadIdx.x; e < ca + cb; e += blockDim.x) out[e] = merged[e];
}

// Lowest stored level: `first`, or the tile stage's top level when merge passes follow and
// read it.
int tree_store_base(int levels, int first) {
    const int top_tile = levels - 1 < kTileLog ? levels - 1 : kTileLog;
    return (top_tile + 1 < levels && first > top_tile) ? top_tile : first;
}

template <typename CT, int S>
static hipError_t build_tree_t(int64_t BH, int64_t N, int levels, int first, const CT* zk,
                               uint64_t* tree_asc, uint64_t* tree_desc, hipStream_t s) {
    if (BH <= 0 || N <= 0) return hipSuccess;
    const int top_tile = levels - 1 < kTileLog ? levels - 1 : kTileLog;
    dim3 grid(static_cast<unsigned>((N + kTile - 1) / kTile), static_cast<unsigned>(BH));
    const int base = tree_store_base(levels, first);
    const int stored = levels > base ? levels - base : 0;
    hipLaunchKernelGGL((zeta_tree_tile_kernel<CT, S>), grid, dim3(kTile), 0, s, zk, tree_asc,
                       tree_desc, N, stored, top_tile, base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    for (int l = top_tile; l + 1 < levels; ++l) {
        dim3 g(static_cast<unsigned>((N + kMergeTile - 1) / kMergeTile),
               static_cast<unsigned>(BH), 2);
        hipLaunchKernelGGL(zeta_tree_merge_kernel, g, dim3(kMergeThreads), 0, s, tree_asc, tree_desc, N,
                           stored, base, l);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_build_tree(int64_t BH, int64_t N, int levels, int first, const uint32_t* zk,
                             uint64_t* tree_asc, uint64_t* tree_desc, hipStream_t s) {
    return build_tree_t<uint32_t, 32>(BH, N, levels, first, zk, tree_asc, tree_desc, s);
}

hipError_t launch_build_tree36(int64_t BH, int64_t N, int levels, int first, const uint64_t* zk,
                               uint64_t* tree_asc, uint64_t* tree_desc, hipStream_t s) {
    return build_tree_t<uint64_t, 28>(BH, N, levels, first, zk, tree_asc, tree_desc, s);
}

}  // namespace zeta
