// Device helpers shared by the HIP translation units of libtq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"

namespace tq {

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
