// probe.hip -- measurement kernel: the rate of scattered row gathers.
//
// The gather and both backward passes spend their time reading whole value (or upstream
// gradient) rows named by the selection: one 16-lane row of a wavefront per query or key,
// 16 bytes per lane, the loads of eight rows issued together.  Those rows are mostly L2 hits
// (queries close on the Z-order curve select the same rows and run together), so the limit
// of these kernels is the rate at which the vector memory pipeline serves such loads, not
// HBM bandwidth.  This kernel measures that rate with the same access shape and no other
// work: every group of 16 lanes reads `rows_per_group` rows drawn uniformly from a table
// (a counter-based hash of the group and the row number), eight rows in flight together, and
// folds the words it loaded into one value per group so that no load is dead.  A table that
// fits in one XCD's L2 gives the L2-resident ceiling; larger tables the Infinity Cache and
// HBM rates.
#include "zeta_internal.hpp"

namespace zeta {

constexpr int kProbeLanes = 16;
constexpr int kProbeLoads = 8;
constexpr int kProbeThreads = 256;

// Counter-based mixing of (group, row number) to a row: the finaliser of the 32-bit
// MurmurHash3 (Appleby), applied to a Weyl sequence of the group's seed.
__device__ __forceinline__ uint32_t probe_mix(uint32_t x) {
    x ^= x >> 16;
    x *= 0x85ebca6bu;
    x ^= x >> 13;
    x *= 0xc2b2ae35u;
    x ^= x >> 16;
    return x;
}

__global__ void __launch_bounds__(kProbeThreads) zeta_probe_row_gather_kernel(
    const uint4* __restrict__ table, uint32_t row_mask, int chunks, int64_t groups,
    int rows_per_group, uint32_t seed, uint32_t* __restrict__ sink) {
    const int64_t g = static_cast<int64_t>(blockIdx.x) * (kProbeThreads / kProbeLanes) +
                      threadIdx.x / kProbeLanes;
    const int lane = threadIdx.x & (kProbeLanes - 1);
    if (g >= groups) return;  // uniform over the group's 16 lanes
    const uint32_t base = probe_mix(seed ^ static_cast<uint32_t>(g) * 0x9e3779b9u);
    const int c = lane < chunks ? lane : chunks - 1;  // rows narrower than 256 B: lanes repeat
    uint32_t fold = 0;
    for (int r0 = 0; r0 < rows_per_group; r0 += kProbeLoads) {
        uint4 v[kProbeLoads];
#pragma unroll
        for (int u = 0; u < kProbeLoads; ++u) {
            const uint32_t row = probe_mix(base + static_cast<uint32_t>(r0 + u)) & row_mask;
            v[u] = table[static_cast<int64_t>(row) * chunks + c];
        }
#pragma unroll
        for (int u = 0; u < kProbeLoads; ++u) fold ^= v[u].x + v[u].y + v[u].z + v[u].w;
    }
    if (lane == 0) sink[g] = fold;
}

hipError_t launch_probe_row_gather(const void* table, int64_t table_rows, int row_bytes,
                                   int64_t groups, int rows_per_group, uint32_t seed,
                                   uint32_t* sink, hipStream_t s) {
    if (groups <= 0) return hipSuccess;
    const int64_t blocks = (groups + kProbeThreads / kProbeLanes - 1) / (kProbeThreads / kProbeLanes);
    hipLaunchKernelGGL(zeta_probe_row_gather_kernel, dim3(static_cast<unsigned>(blocks)),
                       dim3(kProbeThreads), 0, s, static_cast<const uint4*>(table),
                       static_cast<uint32_t>(table_rows - 1), row_bytes / 16, groups,
                       rows_per_group, seed, sink);
    return hipGetLastError();
}

}  // namespace zeta
