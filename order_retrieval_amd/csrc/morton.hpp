// morton.hpp -- the 10-bit-cell Z-order code of one three-dimensional fp32 point.
//
// "ZETA: Leveraging Z-order Curves for Efficient Top-k Attention", rebuttal page, answer
// W2/A2 "Clarification of Binary Expansion and Precision": each coordinate is put on a
// fixed grid and the bits of the three cells are interleaved into one integer.  The grid is
// [-4, 4) with 1024 cells: cell = clamp(floor(128 x) + 512, 0, 1023), NaN -> 0, and bit b of
// axis a becomes bit 3b + a.  128 x is an exact power-of-two scaling in fp32, so floorf sees
// the exact value and the cell is exact.
#pragma once

#include "zeta_internal.hpp"

namespace zeta {

__device__ __forceinline__ uint32_t cell10(float x) {
    if (!(x == x)) return 0u;  // NaN
    x = fminf(fmaxf(x, -4.0f), 4.0f);
    int c = static_cast<int>(floorf(x * 128.0f)) + 512;
    return static_cast<uint32_t>(c > 1023 ? 1023 : c);
}

// Spread the 10 low bits of v so that bit b moves to bit 3b.
__device__ __forceinline__ uint32_t spread3(uint32_t v) {
    v = (v | (v << 16)) & 0x030000FFu;
    v = (v | (v << 8)) & 0x0300F00Fu;
    v = (v | (v << 4)) & 0x030C30C3u;
    v = (v | (v << 2)) & 0x09249249u;
    return v;
}

__device__ __forceinline__ uint32_t morton3(float x0, float x1, float x2) {
    return spread3(cell10(x0)) | (spread3(cell10(x1)) << 1) | (spread3(cell10(x2)) << 2);
}

// Coordinate `a` of the curve's axis order: axis a reads coordinate (perm >> 2a) & 3.
__device__ __forceinline__ float axis_of(float x0, float x1, float x2, int perm, int a) {
    const int c = (perm >> (2 * a)) & 3;
    return c == 0 ? x0 : (c == 1 ? x1 : x2);
}

__device__ __forceinline__ uint32_t morton3p(float x0, float x1, float x2, int perm) {
    return morton3(axis_of(x0, x1, x2, perm, 0), axis_of(x0, x1, x2, perm, 1),
                   axis_of(x0, x1, x2, perm, 2));
}

}  // namespace zeta
