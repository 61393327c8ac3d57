// order.hip -- Z-order processing order for the row-gathering kernels.
//
// Queries whose codes are close select largely the same keys (their neighbourhoods on the
// Z-order line overlap), so processing queries bucketed by the high bits of their code
// makes the value rows that concurrent workgroups read overlap, and an XCD's L2 can serve
// them.  (Keys in the per-key backward pass stay in position order: their records are then
// read as one stream, which measured faster than a code order.)
//
// The order only schedules work: every query or key is still computed exactly once and
// independently, so results do not depend on it.  It is a counting sort by the top
// kOrderBits code bits per (b,h) (order inside a bucket is arbitrary), built with LDS
// integer atomics only.
#include "zeta_internal.hpp"

namespace zeta {

constexpr int kOrderBits = 12;
constexpr int kOrderBuckets = 1 << kOrderBits;
constexpr int kOrderShift = 30 - kOrderBits;  // codes are < 2^30

// One workgroup per (b,h): bucket counts, their exclusive scan and the scatter all run in
// LDS (LDS atomics are cheap even on the crowded buckets near the centre of the code range).
constexpr int kOrderThreads = 1024;
__global__ void __launch_bounds__(kOrderThreads) zeta_order_kernel(const uint32_t* __restrict__ codes,
                                                                    int64_t N,
                                                                    uint32_t* __restrict__ perm) {
    __shared__ uint32_t cnt[kOrderBuckets];
    __shared__ uint32_t part[kOrderThreads];
    constexpr int per = kOrderBuckets / kOrderThreads;
    const int64_t bh = blockIdx.x;
    const uint32_t* c = codes + bh * N;
    uint32_t* out = perm + bh * N;
    constexpr int B8 = 8;  // codes loaded per thread before their atomics (loads in flight)
    for (int b = threadIdx.x; b < kOrderBuckets; b += kOrderThreads) cnt[b] = 0;
    __syncthreads();
    for (int64_t e0 = threadIdx.x; e0 < N; e0 += B8 * kOrderThreads) {
        uint32_t bk[B8];
#pragma unroll
        for (int u = 0; u < B8; ++u) {
            const int64_t e = e0 + u * kOrderThreads;
            bk[u] = e < N ? (c[e] >> kOrderShift) & (kOrderBuckets - 1) : kOrderBuckets;
        }
#pragma unroll
        for (int u = 0; u < B8; ++u)
            if (bk[u] < kOrderBuckets) atomicAdd(&cnt[bk[u]], 1u);
    }
    __syncthreads();
    uint32_t v[per];
    uint32_t sum = 0;
#pragma unroll
    for (int u = 0; u < per; ++u) {
        v[u] = cnt[threadIdx.x * per + u];
        sum += v[u];
    }
    part[threadIdx.x] = sum;
    __syncthreads();
    for (int off = 1; off < kOrderThreads; off <<= 1) {
        const uint32_t y = threadIdx.x >= off ? part[threadIdx.x - off] : 0u;
        __syncthreads();
        part[threadIdx.x] += y;
        __syncthreads();
    }
    uint32_t run = part[threadIdx.x] - sum;
#pragma unroll
    for (int u = 0; u < per; ++u) {
        cnt[threadIdx.x * per + u] = run;
        run += v[u];
    }
    __syncthreads();
    for (int64_t e0 = threadIdx.x; e0 < N; e0 += B8 * kOrderThreads) {
        uint32_t bk[B8];
#pragma unroll
        for (int u = 0; u < B8; ++u) {
            const int64_t e = e0 + u * kOrderThreads;
            bk[u] = e < N ? (c[e] >> kOrderShift) & (kOrderBuckets - 1) : kOrderBuckets;
        }
#pragma unroll
        for (int u = 0; u < B8; ++u) {
            if (bk[u] < kOrderBuckets) {
                const uint32_t pos = atomicAdd(&cnt[bk[u]], 1u);
                out[pos] = static_cast<uint32_t>(e0 + u * kOrderThreads);
            }
        }
    }
}

hipError_t launch_order(int64_t BH, int64_t N, const uint32_t* codes, uint32_t* perm,
                        hipStream_t s) {
    if (BH <= 0 || N <= 0) return hipSuccess;
    hipLaunchKernelGGL(zeta_order_kernel, dim3(static_cast<unsigned>(BH)), dim3(kOrderThreads), 0, s,
                       codes, N, perm);
    return hipGetLastError();
}

}  // namespace zeta
