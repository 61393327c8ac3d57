// order.hip -- Z-order processing order for the row-gathering kernels.
//
// Queries (or keys) whose codes are close select largely the same rows (their neighbourhoods
// on the Z-order line overlap), so processing them bucketed by the high bits of their code
// makes the rows that concurrent workgroups read overlap, and an XCD's L2 can serve them.
// Buckets are fine (12 bits) because normally distributed points crowd the centre cells.
//
// The order only schedules work: every query or key is still computed exactly once and
// independently, so results do not depend on it.  It is a counting sort by the top
// kOrderBits code bits per (b,h) over tiles of kOrderTile positions: per-tile bucket counts
// (tile-major), one scan per (b,h) in (bucket, tile) order, and a scatter that places a
// tile's positions after the earlier tiles' positions of the same bucket (order inside a
// tile's bucket comes from LDS atomics and is arbitrary).
#include "zeta_internal.hpp"
#include "morton.hpp"

namespace zeta {

constexpr int kOrderBits = 12;
constexpr int kOrderBuckets = 1 << kOrderBits;
constexpr int kOrderShift = 30 - kOrderBits;  // codes are < 2^30
constexpr int kOrderThreads = 1024;
constexpr int kOrderPer = kOrderBuckets / kOrderThreads;  // buckets per thread (4: one uint4)
constexpr int kOrderItems = 4;
constexpr int kOrderTile = kOrderThreads * kOrderItems;
static_assert(kOrderPer == 4, "counts move as uint4");
constexpr int kScanChunk = 16;  // tiles whose counts the scan reads at once

int64_t order_tiles(int64_t N) { return (N + kOrderTile - 1) / kOrderTile; }
size_t order_scratch_words(int64_t BH, int64_t N) {
    return static_cast<size_t>(BH * kOrderBuckets * order_tiles(N));
}

__device__ __forceinline__ uint32_t order_bucket(uint32_t code) {
    return (code >> kOrderShift) & (kOrderBuckets - 1);
}

// Bucket counts of one tile: hist[bh][tile][bucket].
__global__ void __launch_bounds__(kOrderThreads) zeta_order_hist_kernel(
    const uint32_t* __restrict__ codes, int64_t N, int64_t tiles, uint4* __restrict__ hist) {
    __shared__ uint32_t cnt[kOrderBuckets];
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < kOrderPer; ++u) cnt[tid * kOrderPer + u] = 0;
    __syncthreads();
    const uint32_t* c = codes + bh * N;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kOrderTile;
    uint32_t bk[kOrderItems];
#pragma unroll
    for (int it = 0; it < kOrderItems; ++it) {
        const int64_t e = t0 + it * kOrderThreads + tid;
        bk[it] = c[e < N ? e : N - 1];  // clamped: the tile's loads issue together
    }
#pragma unroll
    for (int it = 0; it < kOrderItems; ++it) keep(bk[it]);
#pragma unroll
    for (int it = 0; it < kOrderItems; ++it) {
        const int64_t e = t0 + it * kOrderThreads + tid;
        bk[it] = e < N ? order_bucket(bk[it]) : kOrderBuckets;
    }
#pragma unroll
    for (int it = 0; it < kOrderItems; ++it)
        if (bk[it] < kOrderBuckets) atomicAdd(&cnt[bk[it]], 1u);
    __syncthreads();
    hist[(bh * tiles + blockIdx.x) * kOrderThreads + tid] =
        make_uint4(cnt[tid * 4], cnt[tid * 4 + 1], cnt[tid * 4 + 2], cnt[tid * 4 + 3]);
}

// Codes and bucket counts in one pass: one workgroup per tile of kOrderTile positions of a
// (b,h) slice and point set (blockIdx.z: 0 queries, 1 keys).  Each thread encodes four
// consecutive points (three 16-byte loads and one 16-byte store when the slice rows allow)
// and, for a set that gets a processing order, adds their buckets to the tile's counts;
// the counts go to slice set * BH + bh, so keys stored right after the queries are ordered
// by the same scan and scatter as 2 BH slices.
__global__ void __launch_bounds__(kOrderThreads) zeta_encode_hist_kernel(
    const float* __restrict__ q, uint32_t* __restrict__ zq, const float* __restrict__ k,
    uint32_t* __restrict__ zk, int64_t BH, int64_t N, int64_t tiles, int perm, int vec_ok,
    int count_keys, uint4* __restrict__ hist) {
    __shared__ uint32_t cnt[kOrderBuckets];
    const int set = blockIdx.z;
    const float* __restrict__ x = set ? k : q;
    uint32_t* __restrict__ z = set ? zk : zq;
    const bool counted = set == 0 || count_keys != 0;  // uniform over the workgroup
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    if (counted) {
#pragma unroll
        for (int u = 0; u < kOrderPer; ++u) cnt[tid * kOrderPer + u] = 0;
        __syncthreads();
    }
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kOrderTile + tid * 4;  // in the slice
    const int64_t r0 = bh * N + p0;                                              // row
    uint32_t c[4];
    bool ok[4];
    if (vec_ok && p0 + 4 <= N) {  // N % 4 == 0 and aligned bases: row r0 starts a 16-byte word
        const float4* xv = reinterpret_cast<const float4*>(x) + 3 * (r0 / 4);
        const float4 a = xv[0], b = xv[1], d = xv[2];
        c[0] = morton3p(a.x, a.y, a.z, perm);
        c[1] = morton3p(a.w, b.x, b.y, perm);
        c[2] = morton3p(b.z, b.w, d.x, perm);
        c[3] = morton3p(d.y, d.z, d.w, perm);
        *reinterpret_cast<uint4*>(z + r0) = make_uint4(c[0], c[1], c[2], c[3]);
#pragma unroll
        for (int u = 0; u < 4; ++u) ok[u] = true;
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            ok[u] = p0 + u < N;
            c[u] = 0;
            if (ok[u]) {
                const int64_t r = r0 + u;
                c[u] = morton3p(x[3 * r], x[3 * r + 1], x[3 * r + 2], perm);
                z[r] = c[u];
            }
        }
    }
    if (counted) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (ok[u]) atomicAdd(&cnt[order_bucket(c[u])], 1u);
        __syncthreads();
        hist[((set * BH + bh) * tiles + blockIdx.x) * kOrderThreads + tid] =
            make_uint4(cnt[tid * 4], cnt[tid * 4 + 1], cnt[tid * 4 + 2], cnt[tid * 4 + 3]);
    }
}

// Per (b,h): exclusive scan in (bucket, tile) order, in place.  Thread t owns buckets
// 4t .. 4t+3; the tiles' counts of those buckets are one coalesced uint4 per tile.
__global__ void __launch_bounds__(kOrderThreads) zeta_order_scan_kernel(uint4* __restrict__ hist,
                                                                         int64_t tiles) {
    __shared__ uint32_t part[kOrderThreads];
    const int tid = threadIdx.x;
    uint4* h = hist + static_cast<int64_t>(blockIdx.x) * tiles * kOrderThreads + tid;
    // the tiles' counts are read kScanChunk at a time from clamped positions, all in flight
    // together; with at most kScanChunk tiles they stay in registers for the second pass
    uint32_t tot[kOrderPer] = {0, 0, 0, 0};
    uint4 x[kScanChunk];
    for (int64_t t0 = 0; t0 < tiles; t0 += kScanChunk) {
#pragma unroll
        for (int u = 0; u < kScanChunk; ++u) {
            const int64_t t = t0 + u < tiles ? t0 + u : tiles - 1;
            x[u] = h[t * kOrderThreads];
        }
#pragma unroll
        for (int u = 0; u < kScanChunk; ++u) keep(x[u]);
#pragma unroll
        for (int u = 0; u < kScanChunk; ++u) {
            if (t0 + u < tiles) {
                tot[0] += x[u].x;
                tot[1] += x[u].y;
                tot[2] += x[u].z;
                tot[3] += x[u].w;
            }
        }
    }
    const uint32_t mine = tot[0] + tot[1] + tot[2] + tot[3];
    // exclusive scan over the threads: inside each wavefront by shuffles, then over the
    // wavefront totals
    const int lane = tid & 63, wave = tid >> 6;
    uint32_t incl = mine;
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    if (lane == 63) part[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const uint32_t w = lane < kOrderThreads / 64 ? part[lane] : 0u;
        uint32_t wi = w;
        for (int off = 1; off < kOrderThreads / 64; off <<= 1) {
            const uint32_t y = __shfl_up(wi, off, 64);
            if (lane >= off) wi += y;
        }
        if (lane < kOrderThreads / 64) part[lane] = wi - w;  // exclusive wavefront offsets
    }
    __syncthreads();
    uint32_t run[kOrderPer];
    run[0] = part[wave] + incl - mine;
    run[1] = run[0] + tot[0];
    run[2] = run[1] + tot[1];
    run[3] = run[2] + tot[2];
    for (int64_t t0 = 0; t0 < tiles; t0 += kScanChunk) {
        if (tiles > kScanChunk) {
#pragma unroll
            for (int u = 0; u < kScanChunk; ++u) {
                const int64_t t = t0 + u < tiles ? t0 + u : tiles - 1;
                x[u] = h[t * kOrderThreads];
            }
#pragma unroll
            for (int u = 0; u < kScanChunk; ++u) keep(x[u]);
        }
#pragma unroll
        for (int u = 0; u < kScanChunk; ++u) {
            if (t0 + u < tiles) {
                h[(t0 + u) * kOrderThreads] = make_uint4(run[0], run[1], run[2], run[3]);
                run[0] += x[u].x;
                run[1] += x[u].y;
                run[2] += x[u].z;
                run[3] += x[u].w;
            }
        }
    }
}

// Exclusive sum over the workgroup's 1024 threads of one value each (wavefront shuffles,
// then the sixteen wavefront totals in wavefront 0).  `part` holds kOrderThreads / 64 words.
__device__ __forceinline__ uint32_t order_excl_scan(uint32_t mine, uint32_t* part) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t incl = mine;
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    if (lane == 63) part[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const uint32_t w = lane < kOrderThreads / 64 ? part[lane] : 0u;
        uint32_t wi = w;
        for (int off = 1; off < kOrderThreads / 64; off <<= 1) {
            const uint32_t y = __shfl_up(wi, off, 64);
            if (lane >= off) wi += y;
        }
        if (lane < kOrderThreads / 64) part[lane] = wi - w;  // exclusive wavefront offsets
    }
    __syncthreads();
    return part[wave] + incl - mine;
}

// Slices of at most kFuseTiles tiles: the scatter workgroup scans the slice's counts itself
// (every tile's counts of the thread's four buckets, then one workgroup scan), so no scan
// launch runs between the counts and the scatter.
constexpr int64_t kFuseTiles = 32;

// Places every position of a tile at its bucket's next free slot.  SCAN: the counts are
// raw and the workgroup forms its tile's bucket starts from them; otherwise they were
// scanned in place by zeta_order_scan_kernel.
template <bool SCAN>
__global__ void __launch_bounds__(kOrderThreads) zeta_order_scatter_kernel(
    const uint32_t* __restrict__ codes, int64_t N, int64_t tiles, const uint4* __restrict__ hist,
    uint32_t* __restrict__ perm, uint32_t* __restrict__ rank_of, int64_t rank_slices) {
    __shared__ uint32_t base[kOrderBuckets];
    __shared__ uint32_t part[kOrderThreads / 64];
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    if constexpr (SCAN) {
        // bucket 4 tid + u starts after every position of the lower buckets and this
        // bucket's positions in the earlier tiles
        constexpr int kLoads = 8;
        const uint4* h = hist + bh * tiles * kOrderThreads + tid;
        uint32_t tot[kOrderPer] = {0, 0, 0, 0}, pre[kOrderPer] = {0, 0, 0, 0};
        for (int64_t t0 = 0; t0 < tiles; t0 += kLoads) {
            uint4 x[kLoads];
#pragma unroll
            for (int u = 0; u < kLoads; ++u) {
                const int64_t t = t0 + u < tiles ? t0 + u : tiles - 1;
                x[u] = h[t * kOrderThreads];
            }
#pragma unroll
            for (int u = 0; u < kLoads; ++u) keep(x[u]);
#pragma unroll
            for (int u = 0; u < kLoads; ++u) {
                if (t0 + u < tiles) {
                    tot[0] += x[u].x;
                    tot[1] += x[u].y;
                    tot[2] += x[u].z;
                    tot[3] += x[u].w;
                    if (t0 + u < static_cast<int64_t>(blockIdx.x)) {
                        pre[0] += x[u].x;
                        pre[1] += x[u].y;
                        pre[2] += x[u].z;
                        pre[3] += x[u].w;
                    }
                }
            }
        }
        const uint32_t ex = order_excl_scan(tot[0] + tot[1] + tot[2] + tot[3], part);
        base[tid * 4] = ex + pre[0];
        base[tid * 4 + 1] = ex + tot[0] + pre[1];
        base[tid * 4 + 2] = ex + tot[0] + tot[1] + pre[2];
        base[tid * 4 + 3] = ex + tot[0] + tot[1] + tot[2] + pre[3];
    } else {
        const uint4 b4 = hist[(bh * tiles + blockIdx.x) * kOrderThreads + tid];
        base[tid * 4] = b4.x;
        base[tid * 4 + 1] = b4.y;
        base[tid * 4 + 2] = b4.z;
        base[tid * 4 + 3] = b4.w;
    }
    __syncthreads();
    const uint32_t* c = codes + bh * N;
    uint32_t* out = perm + bh * N;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kOrderTile;
    uint32_t bk[kOrderItems];
#pragma unroll
    for (int it = 0; it < kOrderItems; ++it) {
        const int64_t e = t0 + it * kOrderThreads + tid;
        bk[it] = c[e < N ? e : N - 1];  // clamped: the tile's loads issue together
    }
#pragma unroll
    for (int it = 0; it < kOrderItems; ++it) keep(bk[it]);
#pragma unroll
    for (int it = 0; it < kOrderItems; ++it) {
        const int64_t e = t0 + it * kOrderThreads + tid;
        bk[it] = e < N ? order_bucket(bk[it]) : kOrderBuckets;
    }
#pragma unroll
    for (int it = 0; it < kOrderItems; ++it) {
        if (bk[it] < kOrderBuckets) {
            const uint32_t pos = atomicAdd(&base[bk[it]], 1u);
            out[pos] = static_cast<uint32_t>(t0 + it * kOrderThreads + tid);
            // the inverse, position -> rank (consecutive threads write consecutive positions)
            if (bh < rank_slices) rank_of[bh * N + t0 + it * kOrderThreads + tid] = pos;
        }
    }
}

// The scan (in place, unless the scatter does it) and the scatter of `slices` slices whose
// counts are in hist.
static hipError_t order_scan_scatter(int64_t slices, int64_t N, int64_t tiles,
                                     const uint32_t* codes, uint4* hist, uint32_t* perm,
                                     uint32_t* rank_of, int64_t rank_slices, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(slices));
    if (tiles <= kFuseTiles) {
        hipLaunchKernelGGL(zeta_order_scatter_kernel<true>, grid, dim3(kOrderThreads), 0, s, codes,
                           N, tiles, hist, perm, rank_of, rank_slices);
    } else {
        hipLaunchKernelGGL(zeta_order_scan_kernel, dim3(static_cast<unsigned>(slices)),
                           dim3(kOrderThreads), 0, s, hist, tiles);
        hipLaunchKernelGGL(zeta_order_scatter_kernel<false>, grid, dim3(kOrderThreads), 0, s,
                           codes, N, tiles, hist, perm, rank_of, rank_slices);
    }
    return hipGetLastError();
}

hipError_t launch_encode_order(const float* q, uint32_t* zq, const float* k, uint32_t* zk,
                               int64_t BH, int64_t N, int perm, bool order_keys,
                               uint32_t* order, uint32_t* scratch, hipStream_t s,
                               uint32_t* rank_of) {
    if (BH <= 0 || N <= 0) return hipSuccess;
    // the keys' order slices follow the queries': their codes must too
    if (order_keys && zk != zq + BH * N) return hipErrorInvalidValue;
    auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    const int vec_ok = (N % 4 == 0) && a16(q) && a16(zq) && a16(k) && a16(zk);
    const int64_t tiles = order_tiles(N);
    const int64_t slices = order_keys ? 2 * BH : BH;
    uint4* hist = reinterpret_cast<uint4*>(scratch);  // the workspace carve is 256-byte aligned
    hipLaunchKernelGGL(zeta_encode_hist_kernel,
                       dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(BH), 2u),
                       dim3(kOrderThreads), 0, s, q, zq, k, zk, BH, N, tiles, perm, vec_ok,
                       order_keys ? 1 : 0, hist);
    return order_scan_scatter(slices, N, tiles, zq, hist, order, rank_of, rank_of ? BH : 0, s);
}

hipError_t launch_order(int64_t BH, int64_t N, const uint32_t* codes, uint32_t* perm,
                        uint32_t* scratch, hipStream_t s) {
    if (BH <= 0 || N <= 0) return hipSuccess;
    const int64_t tiles = order_tiles(N);
    const dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(BH));
    uint4* hist = reinterpret_cast<uint4*>(scratch);  // the workspace carve is 256-byte aligned
    hipLaunchKernelGGL(zeta_order_hist_kernel, grid, dim3(kOrderThreads), 0, s, codes, N, tiles,
                       hist);
    return order_scan_scatter(BH, N, tiles, codes, hist, perm, nullptr, 0, s);
}

}  // namespace zeta
