// Device helpers shared by the HIP translation units of libtq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

#include "tq_internal.h"

namespace tq {

constexpr float kLog2e = 1.4426950408889634f;

// Lane exchange inside a row of 16 lanes through DPP (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

__device__ __forceinline__ float lane_value(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// Maximum / sum over the 64 lanes; every lane receives the same value (the
// butterfly is symmetric, so the sum is bit-identical in all lanes).
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<kDppXor1>(x));
    x = fmaxf(x, dpp<kDppXor2>(x));
    x = fmaxf(x, dpp<kDppHalfMirror>(x));
    x = fmaxf(x, dpp<kDppMirror>(x));
    return fmaxf(fmaxf(lane_value(x, 0), lane_value(x, 16)), fmaxf(lane_value(x, 32), lane_value(x, 48)));
}

__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppHalfMirror>(x);
    x += dpp<kDppMirror>(x);
    return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}

// Unnormalized Sylvester Walsh-Hadamard transform of a vector spread over one
// wavefront: element j = DPL * lane + k sits in v[k].
template <int DPL>
__device__ __forceinline__ void wht_wave(float (&v)[DPL], int lane) {
#pragma unroll
    for (int st = 1; st < DPL; st <<= 1)
#pragma unroll
        for (int k = 0; k < DPL; ++k)
            if ((k & st) == 0) {
                const float x = v[k], y = v[k + st];
                v[k] = x + y;
                v[k + st] = x - y;
            }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int k = 0; k < DPL; ++k) {
            const float p = __shfl_xor(v[k], m, 64);
            v[k] = upper ? (p - v[k]) : (v[k] + p);
        }
    }
}

template <int... I, typename F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    _Float16 h;
    const uint16_t b = static_cast<uint16_t>(bits16);
    __builtin_memcpy(&h, &b, 2);
    return static_cast<float>(h);
}

// Round to nearest even fp16, returned as its bit pattern.
__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
    const _Float16 h = static_cast<_Float16>(f);
    uint16_t b;
    __builtin_memcpy(&b, &h, 2);
    return b;
}

__device__ __forceinline__ float rotation_sign(const DevCodebook& cb, int j) {
    return ((cb.sign_bits[j >> 5] >> (j & 31)) & 1u) ? -1.0f : 1.0f;
}

// Walsh-Hadamard butterflies over a vector spread as 8 consecutive elements
// per lane across LPV lanes (element j = 8*lane + e).  In-lane stages cover
// index bits 0..2, lane exchanges cover the rest.  Unnormalized: v <- H v.
template <int LPV>
__device__ __forceinline__ void wht8(float (&v)[8], int lane_in_vec) {
#pragma unroll
    for (int s = 1; s < 8; s <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if ((e & s) == 0) {
                const float a = v[e], b = v[e + s];
                v[e] = a + b;
                v[e + s] = a - b;
            }
        }
    }
#pragma unroll
    for (int m = 1; m < LPV; m <<= 1) {
        const bool upper = (lane_in_vec & m) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = __shfl_xor(v[e], m, LPV);
            v[e] = upper ? (p - v[e]) : (v[e] + p);
        }
    }
}

template <int LPV>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = 1; m < LPV; m <<= 1) x += __shfl_xor(x, m, LPV);
    return x;
}

}  // namespace tq
