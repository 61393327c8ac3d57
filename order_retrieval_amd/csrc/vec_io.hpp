// vec_io.hpp -- 16-byte row-chunk loads/stores of fp32 or bf16 value rows as fp32.
#pragma once

#include "zeta_internal.hpp"

namespace zeta {

template <bool BF16>
struct VecIO;

// A row of a (b,h) slice is named by a 32-bit value that the lane owning it broadcasts: its
// byte offset from the slice base when every row of the slice lies within 2 GiB of it (O32;
// the load is then a uniform base plus a 32-bit offset), else its index.
template <bool BF16, bool O32>
struct RowRef;

template <>
struct VecIO<true> {
    using elem_t = uint16_t;
    using raw_t = uint4;  // the chunk as loaded (unpacked only where it is used)
    static constexpr int kElems = 8;
    __device__ __forceinline__ static raw_t load_raw(const uint16_t* p) {
        return *reinterpret_cast<const uint4*>(p);
    }
    // the chunk at byte offset `off` from `base` (a uniform base plus a 32-bit vector offset)
    __device__ __forceinline__ static raw_t load_raw_at(const uint16_t* base, uint32_t off) {
        return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + off);
    }
    __device__ __forceinline__ static void unpack(const raw_t& u, float (&x)[8]) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            x[2 * t] = __uint_as_float(w[t] << 16);
            x[2 * t + 1] = __uint_as_float(w[t] & 0xffff0000u);
        }
    }
    __device__ __forceinline__ static void load(const uint16_t* p, float (&x)[8]) {
        unpack(load_raw(p), x);
    }
    __device__ __forceinline__ static void store(uint16_t* p, const float (&x)[8]) {
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            w[t] = static_cast<uint32_t>(f32_to_bf16(x[2 * t])) |
                   (static_cast<uint32_t>(f32_to_bf16(x[2 * t + 1])) << 16);
        *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
};

template <>
struct VecIO<false> {
    using elem_t = float;
    using raw_t = float4;
    static constexpr int kElems = 4;
    __device__ __forceinline__ static raw_t load_raw(const float* p) {
        return *reinterpret_cast<const float4*>(p);
    }
    __device__ __forceinline__ static raw_t load_raw_at(const float* base, uint32_t off) {
        return *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(base) + off);
    }
    __device__ __forceinline__ static void unpack(const raw_t& u, float (&x)[4]) {
        x[0] = u.x;
        x[1] = u.y;
        x[2] = u.z;
        x[3] = u.w;
    }
    __device__ __forceinline__ static void load(const float* p, float (&x)[4]) {
        unpack(load_raw(p), x);
    }
    __device__ __forceinline__ static void store(float* p, const float (&x)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    }
};

template <bool BF16, bool O32>
struct RowRef {
    using IO = VecIO<BF16>;
    using T = typename IO::elem_t;
    // name of row r (r < rows of the slice); `dv` elements per row
    __device__ __forceinline__ static uint32_t name(int64_t r, int dv) {
        return O32 ? static_cast<uint32_t>(r) * static_cast<uint32_t>(dv * sizeof(T))
                   : static_cast<uint32_t>(r);
    }
    // the lane's chunk at element offset `coff` of the named row
    __device__ __forceinline__ static typename IO::raw_t load(const T* base, uint32_t nm, int dv,
                                                              int coff) {
        if constexpr (O32)
            return IO::load_raw_at(base, nm + static_cast<uint32_t>(coff * sizeof(T)));
        else
            return IO::load_raw(base + static_cast<int64_t>(nm) * dv + coff);
    }
};

// True when every row of an N x dv slice of `esize`-byte elements lies within 2 GiB of the
// slice base (32-bit row offsets).
inline bool rows_fit_32(int64_t N, int64_t dv, int64_t esize) {
    return N * dv * esize < (int64_t(1) << 31);
}

}  // namespace zeta
