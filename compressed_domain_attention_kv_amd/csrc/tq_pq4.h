// PQ4 encoding of one fp16 row spread over a group of lanes (gfx950), shared by
// the write kernel and the decode kernel that appends a step's token itself, so
// both write the same bytes.  [P1] "turbo4 post-mortem", section 5: fp16 norm,
// rotation, nearest of 16 centroids, two codes per byte.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_device.h"

namespace tq {

constexpr int kDppQuadRev = 0x1B;  // quad_perm [3,2,1,0]

// DPP move with bound_ctrl set (every pattern used here stays inside its row, so it
// changes nothing), which lets the compiler fold the move into the VALU op using it
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// value of lane l ^ M (M = 1, 2, 4, 8) inside each row of 16 lanes, by DPP moves
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
    if constexpr (M == 1) return dpp_f<kDppXor1>(x);
    else if constexpr (M == 2) return dpp_f<kDppXor2>(x);
    else if constexpr (M == 4) return dpp_f<kDppQuadRev>(dpp_f<kDppHalfMirror>(x));  // 7 - (l ^ 3) = l ^ 4
    else return dpp_f<kDppHalfMirror>(dpp_f<kDppMirror>(x));                       // 15 - (l ^ 7) = l ^ 8
}

// The code of y for 16 sorted boundaries by binary search: four comparisons,
// each against the boundary the earlier ones select (b[7]; b[c + 3]; b[c + 1];
// b[c]), so strict comparisons in fp32 give exactly #{k : b[k] < y}.  The first
// two come from registers; the quad b[c .. c+3] holding the last two candidates
// is one LDS read (a select among four or eight register values is turned into a
// lookup table in scratch memory by the compiler).
__device__ __forceinline__ uint32_t code_of16(float y, float b3, float b7, float b11, const float4* sb4) {
    const bool m8 = y > b7;
    const bool m4 = y > (m8 ? b11 : b3);
    const uint32_t q = (m8 ? 2u : 0u) | (m4 ? 1u : 0u);
    const float4 f = sb4[q];
    const bool m2 = y > f.y;
    const bool m1 = y > (m2 ? f.z : f.x);
    return 4u * q | (m2 ? 2u : 0u) | (m1 ? 1u : 0u);
}

// The rotation signs of a lane's CPL coordinates (bit e for its coordinate e) as XOR masks
// of its fp16 input words (bit 15 / 31 per coordinate).
template <int CPL>
__device__ __forceinline__ void pq4_sign_masks(uint32_t sgn, uint32_t (&smask)[CPL / 2]) {
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i) smask[i] = (((sgn >> (2 * i)) & 1u) << 15) | (((sgn >> (2 * i + 1)) & 1u) << 31);
}

// One row: lane l of the LANES lanes of the row (lanes l ^ 1 .. l ^ 8 of one DPP row)
// holds its CPL fp16 inputs in raw; returns the fp16 norm bits and the lane's CPL / 8
// code words.  Steps: s * x (sign-bit flips), norm over the lanes, u = x / n scaled by
// 1/sqrt(d), y = H (s * u) with stages over index bits 0 .. log2(d) - 1 in order, codes.
template <int D, int LANES>
__device__ __forceinline__ void pq4_encode(const uint4 (&raw)[D / LANES / 8], const uint32_t (&smask)[D / LANES / 2],
                                           float b3, float b7, float b11, const float4* sb4, int l, uint32_t& n16,
                                           uint32_t (&words)[D / LANES / 8]) {
    constexpr int CPL = D / LANES, NPC = CPL / 8;
    constexpr float kInvSqrtD = D == 256 ? 0.0625f : 0.08838834764831845f;
    float v[CPL];
#pragma unroll
    for (int c = 0; c < NPC; ++c) {
        const uint32_t w[4] = {raw[c].x ^ smask[4 * c], raw[c].y ^ smask[4 * c + 1], raw[c].z ^ smask[4 * c + 2],
                               raw[c].w ^ smask[4 * c + 3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * c + e] = half_bits_to_float((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    }
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) ss += v[e] * v[e];
    static_for<__builtin_ctz(LANES)>([&](auto mc) { ss += lane_xor<(1 << decltype(mc)::value)>(ss); });
    const float n = sqrtf(ss);
    n16 = float_to_half_bits(fminf(n, kFp16Max));
    const float scale = (n > 0.0f ? __fdiv_rn(1.0f, n) : 0.0f) * kInvSqrtD;  // 1 / (n sqrt(d))
#pragma unroll
    for (int e = 0; e < CPL; ++e) v[e] *= scale;
#pragma unroll
    for (int st = 1; st < CPL; st <<= 1)
#pragma unroll
        for (int e = 0; e < CPL; ++e)
            if ((e & st) == 0) {
                const float x = v[e], y = v[e + st];
                v[e] = x + y;
                v[e + st] = x - y;
            }
    static_for<__builtin_ctz(LANES)>([&](auto mc) {
        constexpr int M = 1 << decltype(mc)::value;
        const bool upper = (l & M) != 0;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const float p = lane_xor<M>(v[e]);
            v[e] = upper ? (p - v[e]) : (v[e] + p);
        }
    });
#pragma unroll
    for (int wq = 0; wq < CPL / 8; ++wq) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) word |= code_of16(v[8 * wq + e], b3, b7, b11, sb4) << (4 * e);
        words[wq] = word;
    }
}

// Lane l's part of the row's 68-byte blocks at out: coordinates CPL l .. lie in block
// (CPL l) / 128, their codes from byte 4 + (CPL l % 128) / 2; the lane that starts a
// block also writes its [fp16 norm][2 zero bytes].  A row starts at a multiple of 68
// bytes, so only 4-byte alignment is known: the code words are stored as dwords (the
// compiler joins them into one wide store, which the hardware allows at that alignment).
template <int D, int LANES>
__device__ __forceinline__ void pq4_store(uint8_t* out, int l, uint32_t n16, const uint32_t (&words)[D / LANES / 8]) {
    constexpr int CPL = D / LANES;
    uint8_t* bp = out + 68 * ((CPL * l) / 128);
    const int cofs = 4 + ((CPL * l) % 128) / 2;
    if ((CPL * l) % 128 == 0) *reinterpret_cast<uint32_t*>(bp) = n16;
    uint32_t* cw = reinterpret_cast<uint32_t*>(bp + cofs);
#pragma unroll
    for (int i = 0; i < CPL / 8; ++i) cw[i] = words[i];
}

}  // namespace tq
