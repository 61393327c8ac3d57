// vec_io.hpp -- 16-byte row-chunk loads/stores of fp32 or bf16 value rows as fp32.
#pragma once

#include "zeta_internal.hpp"

namespace zeta {

template <bool BF16>
struct VecIO;

template <>
struct VecIO<true> {
    using elem_t = uint16_t;
    using raw_t = uint4;  // the chunk as loaded (unpacked only where it is used)
    static constexpr int kElems = 8;
    __device__ __forceinline__ static raw_t load_raw(const uint16_t* p) {
        return *reinterpret_cast<const uint4*>(p);
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

}  // namespace zeta
