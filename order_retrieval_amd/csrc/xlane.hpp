// xlane.hpp -- cross-lane sums inside a wavefront.
#pragma once

#include <type_traits>

#include "zeta_internal.hpp"

namespace zeta {

// x from another lane of the same 16-lane row, by a DPP pattern (a modifier of the VALU
// instruction that reads it, no LDS round trip).  Every lane is active where these are used,
// and every pattern here reads a lane of the same row, so no lane ever takes the zero that
// bound_ctrl supplies for a missing source; setting it lets the compiler fold the move into
// the instruction that consumes it (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp_take(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane l of an 8-lane half-row takes lane 7-l
constexpr int kDppMirror = 0x140;      // lane l of a 16-lane row takes lane 15-l

// f(std::integral_constant<int, I>{}) for I = B .. E-1, each I a compile-time constant.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Every lane of a 16-lane row takes lane L of that row (DPP row_newbcast).
template <int L>
__device__ __forceinline__ float row_bcast(float x) {
    static_assert(L >= 0 && L < 16, "a row has 16 lanes");
    return dpp_take<0x150 + L>(x);
}
template <int L>
__device__ __forceinline__ uint32_t row_bcast(uint32_t x) {
    static_assert(L >= 0 && L < 16, "a row has 16 lanes");
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x150 + L, 0xF, 0xF, true));
}

// Reduce-scatter of 8 slots over a 16-lane row: v[s] is this lane's part of slot s's sum;
// lanes 2s and 2s + 1 of the row return the row's total of slot s.  Three exchange steps,
// with the partners 15 - l, then 7 - l inside the half-row, then l ^ 2 (their lowest
// differing lane bits are 3, 2, 1), each halve the slots a lane holds: it keeps the half whose
// slot bit equals its lane bit and adds the partner's part of it; a last add with lane l ^ 1
// joins the two halves of the row.  The summation order is fixed, so the result is
// reproducible.  22 VALU instructions for 8 slots (a group_sum per slot takes 32, in longer
// dependent chains).
__device__ __forceinline__ float row_reduce_scatter8(const float (&v)[8], int lrow) {
    float a[4], b[2];
    const bool b3 = (lrow & 8) != 0, b2 = (lrow & 4) != 0, b1 = (lrow & 2) != 0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        a[k] = (b3 ? v[4 + k] : v[k]) + dpp_take<kDppMirror>(b3 ? v[k] : v[4 + k]);
#pragma unroll
    for (int k = 0; k < 2; ++k)
        b[k] = (b2 ? a[2 + k] : a[k]) + dpp_take<kDppHalfMirror>(b2 ? a[k] : a[2 + k]);
    const float c = (b1 ? b[1] : b[0]) + dpp_take<kDppXor2>(b1 ? b[0] : b[1]);
    return c + dpp_take<kDppXor1>(c);
}

// Sum over aligned groups of G lanes (G a power of two, 8 <= G <= 64).  Each step adds the
// partner block's partial sum: partners xor 1 and xor 2 inside a quad, then the mirrored
// quad of the half-row and the mirrored half of the row, then xor 16 and xor 32 across rows.
// Since a + b == b + a exactly, every lane of a group ends with the same bits.
__device__ __forceinline__ float group_sum(float x, int G) {
    x += dpp_take<kDppXor1>(x);
    x += dpp_take<kDppXor2>(x);
    x += dpp_take<kDppHalfMirror>(x);
    if (G > 8) x += dpp_take<kDppMirror>(x);
    for (int off = 16; off < G; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Lanes of the wavefront whose B-bit digit equals this lane's, among the valid ones: the AND
// over the digit's bits of the ballot of that bit (or of its complement where the lane's bit
// is 0).  Each bit's 0 / all-ones mask is a sign-extended bit field, so a bit costs a compare,
// a field extract and an xor per 32-bit half (gfx950 folds the AND into v_bitop3).  With the
// lanes below this one masked off, the popcount is the lane's stable rank among its peers.
template <int B>
__device__ __forceinline__ uint64_t digit_peers(uint32_t digit, bool valid) {
    const uint64_t v = __ballot(valid);
    uint32_t lo = valid ? static_cast<uint32_t>(v) : 0u;
    uint32_t hi = valid ? static_cast<uint32_t>(v >> 32) : 0u;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const uint32_t m = static_cast<uint32_t>(static_cast<int32_t>(digit << (31 - b)) >> 31);
        const uint64_t bal = __ballot(m != 0u);
        lo &= ~(static_cast<uint32_t>(bal) ^ m);
        hi &= ~(static_cast<uint32_t>(bal >> 32) ^ m);
    }
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

}  // namespace zeta
