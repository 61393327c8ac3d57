// encode.hip -- Z-order (Morton) code of three-dimensional fp32 points.
//
// "ZETA: Leveraging Z-order Curves for Efficient Top-k Attention", rebuttal page, answer
// W2/A2 "Clarification of Binary Expansion and Precision": each coordinate is put on a
// fixed grid and the bits of the three cells are interleaved into one integer.  Here the
// grid is [-4, 4) with 1024 cells: cell = clamp(floor(128 x) + 512, 0, 1023), NaN -> 0,
// and bit b of axis a becomes bit 3b + a.  128 x is an exact power-of-two scaling in fp32,
// so floorf sees the exact value and the cell is exact.
//
// Memory-bound elementwise kernel: 12 B in, 4 B out per point.  Each thread converts four
// consecutive points with three 16-byte loads and one 16-byte store.
#include "zeta_internal.hpp"
#include "morton.hpp"

namespace zeta {

// perm packs the curve's coordinate order (several-curve variant, rebuttal page on the
// asymmetry of interleaving: the coordinates are fed to the curve in a permuted order);
// kPermIdentity = axis a reads coordinate a.
// blockIdx.y selects the point set: (x, z), or (x1, z1) for the second of two encoded in
// one launch (queries and keys).
__global__ void __launch_bounds__(256) zeta_morton_encode_kernel(const float* __restrict__ x0,
                                                                  int64_t rows,
                                                                  uint32_t* __restrict__ z0,
                                                                  int vec_ok, int perm,
                                                                  const float* __restrict__ x1,
                                                                  uint32_t* __restrict__ z1) {
    const float* __restrict__ x = blockIdx.y ? x1 : x0;
    uint32_t* __restrict__ z = blockIdx.y ? z1 : z0;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t r0 = t * 4;
    if (r0 >= rows) return;
    if (vec_ok && r0 + 4 <= rows) {
        const float4* xv = reinterpret_cast<const float4*>(x) + 3 * t;
        float4 a = xv[0], b = xv[1], c = xv[2];
        uint4 o;
        o.x = morton3p(a.x, a.y, a.z, perm);
        o.y = morton3p(a.w, b.x, b.y, perm);
        o.z = morton3p(b.z, b.w, c.x, perm);
        o.w = morton3p(c.y, c.z, c.w, perm);
        *reinterpret_cast<uint4*>(z + r0) = o;
    } else {
        for (int64_t r = r0; r < rows && r < r0 + 4; ++r)
            z[r] = morton3p(x[3 * r], x[3 * r + 1], x[3 * r + 2], perm);
    }
}

static hipError_t encode_sets(const float* x0, uint32_t* z0, const float* x1, uint32_t* z1,
                              int64_t rows, int perm, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    const int vec_ok = a16(x0) && a16(z0) && (!x1 || (a16(x1) && a16(z1)));
    const int64_t threads = (rows + 3) / 4;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(zeta_morton_encode_kernel,
                       dim3(static_cast<unsigned>(blocks), x1 ? 2u : 1u), dim3(256), 0, s, x0,
                       rows, z0, vec_ok, perm, x1, z1);
    return hipGetLastError();
}

hipError_t launch_encode_perm(const float* x, int64_t rows, int perm, uint32_t* z,
                              hipStream_t s) {
    return encode_sets(x, z, nullptr, nullptr, rows, perm, s);
}

hipError_t launch_encode2_perm(const float* q, uint32_t* zq, const float* k, uint32_t* zk,
                               int64_t rows, int perm, hipStream_t s) {
    return encode_sets(q, zq, k, zk, rows, perm, s);
}

// 12-bit cells (rebuttal page, answer W2/A2: a grid of 4096 cells per coordinate, three
// 12-bit components interleaved into 36 bits held in a 64-bit integer).  Same fixed range
// [-4, 4): cell = clamp(floor(512 x) + 2048, 0, 4095), NaN -> 0 (512 x is exact in fp32).
__device__ __forceinline__ uint32_t cell12(float x) {
    if (!(x == x)) return 0u;  // NaN
    x = fminf(fmaxf(x, -4.0f), 4.0f);
    int c = static_cast<int>(floorf(x * 512.0f)) + 2048;
    return static_cast<uint32_t>(c > 4095 ? 4095 : c);
}

// Bit b of a 12-bit cell -> bit 3b (the low 10 bits as for 10-bit cells, then bits 10, 11).
__device__ __forceinline__ uint64_t spread3_12(uint32_t v) {
    return static_cast<uint64_t>(spread3(v & 1023u)) |
           (static_cast<uint64_t>((v >> 10) & 1u) << 30) |
           (static_cast<uint64_t>((v >> 11) & 1u) << 33);
}

__device__ __forceinline__ uint64_t morton3_12(float x0, float x1, float x2) {
    return spread3_12(cell12(x0)) | (spread3_12(cell12(x1)) << 1) | (spread3_12(cell12(x2)) << 2);
}

__global__ void __launch_bounds__(256) zeta_morton36_encode_kernel(const float* __restrict__ x,
                                                                    int64_t rows,
                                                                    uint64_t* __restrict__ z,
                                                                    int perm) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    const float x0 = x[3 * r], x1 = x[3 * r + 1], x2 = x[3 * r + 2];
    z[r] = morton3_12(axis_of(x0, x1, x2, perm, 0), axis_of(x0, x1, x2, perm, 1),
                      axis_of(x0, x1, x2, perm, 2));
}

hipError_t launch_encode36_perm(const float* x, int64_t rows, int perm, uint64_t* z,
                                hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(zeta_morton36_encode_kernel, dim3(static_cast<unsigned>((rows + 255) / 256)),
                       dim3(256), 0, s, x, rows, z, perm);
    return hipGetLastError();
}

hipError_t launch_encode(const float* x, int64_t rows, uint32_t* z, hipStream_t s) {
    return launch_encode_perm(x, rows, kPermIdentity, z, s);
}

}  // namespace zeta
