// Read path of libtq on gfx950: fused decode attention over compressed KV.
//
// decode_partial: one workgroup of 4 wavefronts per (batch row, KV head,
// context split).  Each wavefront walks 64-token tiles of its split:
//   1. the tile's K and V bytes are copied HBM -> LDS with 16-byte loads
//      (a 64-token tile of any format is a 16-byte aligned byte run);
//   2. score phase, one lane per token: the lane decodes its key's codes in
//      registers, looks centroids up in an LDS table and accumulates
//      q_rot[j] * c[code_j] for every query head of the group (the rotated
//      query sits in LDS, pre-scaled by log2(e)/sqrt(d)); TQ3K adds the QJL
//      term; the block norm scales the sum;
//   3. online softmax per query head across the wavefront (max/sum by lane
//      exchange), probabilities to LDS;
//   4. value phase, one lane per d/64 coordinates: each token's value codes
//      are decoded in registers and accumulated for every head.
// The four wavefronts' (m, l, acc) are merged in LDS and written as one
// split record.  decode_combine merges the splits of one (b, query head),
// normalizes and, for rotated value formats, applies Pi^T once.

#include <hip/hip_runtime.h>

#include <cmath>
#include <utility>

#include "tq_device.h"

namespace tq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int FMT, int D>
constexpr int vbytes() {
    return FMT == TQ_FMT_PQ4 ? 68 * (D / 128)
         : FMT == TQ_FMT_PQ3 ? 14 * (D / 32)
         : FMT == TQ_FMT_TQ3K ? 4 + D / 4 + D / 8
                              : 12 * (D / kGroup);
}

struct DecodeArgs {
    const float* q_rot;
    const float* q_sk;
    const uint8_t* k_cache;
    const uint8_t* v_cache;
    const int32_t* seq_lens;
    float* scores;
    float2* ml;
    float* acc;
    int hq;
    int hkv;
    int capacity;
    int splits;
    int split_len;
};

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

// byte k of a register-resident little-endian byte run (k known at compile time after unrolling)
template <int N>
__device__ __forceinline__ uint32_t byte_at(const uint32_t (&w)[N], int k) {
    return (w[k >> 2] >> (8 * (k & 3))) & 0xFFu;
}

template <int KF, int VF, int D, int G>
struct Smem {
    static constexpr int VBK = vbytes<KF, D>();
    static constexpr int VBV = vbytes<VF, D>();
    static constexpr bool kSketch = KF == TQ_FMT_TQ3K;
    float q[G * D];                     // rotated query, scaled
    alignas(16) float qs[kSketch ? G * D : 4];  // QJL sketch, scaled
    float2 kpair[256];                  // byte -> (c[lo nibble], c[hi nibble]) for 4-bit keys
    float2 vpair[256];
    float ktab[16];
    float vtab[16];
    alignas(16) uint8_t ktile[kWaves][kTile * VBK];
    alignas(16) uint8_t vtile[kWaves][kTile * VBV];
    float pw[kWaves][kTile * G];        // probabilities of the current tile
};

template <int KF, int VF, int D, int G>
__global__ __launch_bounds__(kWaves * 64) void decode_partial_kernel(DecodeArgs a, DevCodebook cbk, DevCodebook cbv) {
    using SM = Smem<KF, VF, D, G>;
    constexpr int VBK = SM::VBK, VBV = SM::VBV;
    constexpr int DPL = D / 64;  // value coordinates per lane
    __shared__ __align__(16) SM sm;

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int hq0 = h * G;
    int N = a.seq_lens[b];
    N = N < 0 ? 0 : (N > a.capacity ? a.capacity : N);
    const int start = s * a.split_len;
    const int end = min(start + a.split_len, N);
    const size_t rec0 = (static_cast<size_t>(b) * a.hq + hq0) * a.splits + s;  // record of query head hq0

    if (start >= end) {  // empty split: (m, l, acc) = (-inf, 0, 0)
        for (int g = 0; g < G; ++g) {
            const size_t rec = rec0 + static_cast<size_t>(g) * a.splits;
            if (tid == 0) a.ml[rec] = make_float2(-INFINITY, 0.0f);
            for (int j = tid; j < D; j += blockDim.x) a.acc[rec * D + j] = 0.0f;
        }
        return;
    }

    // ---- setup: scaled query, centroid tables
    const float qscale = kLog2e / sqrtf(static_cast<float>(D));
    {
        const float* qg = a.q_rot + (static_cast<size_t>(b) * a.hq + hq0) * D;
        for (int i = tid; i < G * D; i += blockDim.x) sm.q[i] = qg[i] * qscale;
        if constexpr (SM::kSketch) {
            const float kq = qscale * (1.2533141373155003f / D);  // sqrt(pi/2)/d
            const float* sg = a.q_sk + (static_cast<size_t>(b) * a.hq + hq0) * D;
            for (int i = tid; i < G * D; i += blockDim.x) sm.qs[i] = sg[i] * kq;
        }
        if (tid < 16) {
            sm.ktab[tid] = cbk.centroids[tid];
            sm.vtab[tid] = cbv.centroids[tid];
        }
        sm.kpair[tid] = make_float2(cbk.centroids[tid & 15], cbk.centroids[tid >> 4]);
        sm.vpair[tid] = make_float2(cbv.centroids[tid & 15], cbv.centroids[tid >> 4]);
    }
    __syncthreads();

    float m_run[G], l_run[G], acc[G][DPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m_run[g] = -INFINITY;
        l_run[g] = 0.0f;
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[g][k] = 0.0f;
    }

    const size_t stream_row = (static_cast<size_t>(b) * a.hkv + h) * a.capacity;
    const uint8_t* kstream = a.k_cache + stream_row * VBK;
    const uint8_t* vstream = a.v_cache + stream_row * VBV;
    const int trips = (end - start + kSplitQuantum - 1) / kSplitQuantum;

    for (int it = 0; it < trips; ++it) {
        const int t0 = start + it * kSplitQuantum + w * kTile;
        const int nv = max(0, min(kTile, end - t0));

        // ---- 1. stage the tile (in bounds: t0 + 64 <= capacity whenever nv > 0)
        if (nv > 0) {
            const uint4* ks = reinterpret_cast<const uint4*>(kstream + static_cast<size_t>(t0) * VBK);
            const uint4* vs = reinterpret_cast<const uint4*>(vstream + static_cast<size_t>(t0) * VBV);
            uint4* kd = reinterpret_cast<uint4*>(sm.ktile[w]);
            uint4* vd = reinterpret_cast<uint4*>(sm.vtile[w]);
            constexpr int CK = kTile * VBK / 16, CV = kTile * VBV / 16;
#pragma unroll
            for (int c = lane; c < CK; c += 64) kd[c] = ks[c];
#pragma unroll
            for (int c = lane; c < CV; c += 64) vd[c] = vs[c];
        }
        __syncthreads();

        if (nv > 0) {
            // ---- 2. scores, one lane per token
            float t[G];
#pragma unroll
            for (int g = 0; g < G; ++g) t[g] = 0.0f;
            const bool valid = lane < nv;
            const uint8_t* kb = sm.ktile[w] + lane * VBK;
            if constexpr (KF == TQ_FMT_PQ4) {
#pragma unroll
                for (int blk = 0; blk < D / 128; ++blk) {
                    const uint32_t* kw = reinterpret_cast<const uint32_t*>(kb + 68 * blk);
                    const float n = half_bits_to_float(kw[0] & 0xFFFFu);
                    float part[G];
#pragma unroll
                    for (int g = 0; g < G; ++g) part[g] = 0.0f;
#pragma unroll 2
                    for (int dw = 0; dw < 16; ++dw) {
                        const uint32_t word = kw[1 + dw];
#pragma unroll
                        for (int by = 0; by < 4; ++by) {
                            const float2 c = sm.kpair[(word >> (8 * by)) & 0xFFu];
                            const int j = 128 * blk + 8 * dw + 2 * by;
#pragma unroll
                            for (int g = 0; g < G; ++g) {
                                const float2 qq = *reinterpret_cast<const float2*>(&sm.q[g * D + j]);
                                part[g] = fmaf(qq.x, c.x, part[g]);
                                part[g] = fmaf(qq.y, c.y, part[g]);
                            }
                        }
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g) t[g] = fmaf(n, part[g], t[g]);
                }
            } else if constexpr (KF == TQ_FMT_PQ3) {
                constexpr int NW = VBK / 4;
                uint32_t kwv[NW];
#pragma unroll
                for (int i = 0; i < NW; ++i) kwv[i] = reinterpret_cast<const uint32_t*>(kb)[i];
#pragma unroll
                for (int blk = 0; blk < D / 32; ++blk) {
                    const int base = 14 * blk;
                    const float n = half_bits_to_float(byte_at(kwv, base) | (byte_at(kwv, base + 1) << 8));
                    float part[G];
#pragma unroll
                    for (int g = 0; g < G; ++g) part[g] = 0.0f;
#pragma unroll 8
                    for (int jb = 0; jb < 32; ++jb) {
                        const uint32_t lo = (byte_at(kwv, base + 2 + jb / 4) >> (2 * (jb % 4))) & 3u;
                        const uint32_t hi = (byte_at(kwv, base + 10 + jb / 8) >> (jb % 8)) & 1u;
                        const float c = sm.ktab[lo | (hi << 2)];
                        const int j = 32 * blk + jb;
#pragma unroll
                        for (int g = 0; g < G; ++g) part[g] = fmaf(sm.q[g * D + j], c, part[g]);
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g) t[g] = fmaf(n, part[g], t[g]);
                }
            } else {  // TQ3K
                constexpr int NW = VBK / 4;
                uint32_t kwv[NW];
#pragma unroll
                for (int i = 0; i < NW; ++i) kwv[i] = reinterpret_cast<const uint32_t*>(kb)[i];
                const float n = half_bits_to_float(kwv[0] & 0xFFFFu);
                const float gam = half_bits_to_float(kwv[0] >> 16);
                float mse[G], qjl[G];
#pragma unroll
                for (int g = 0; g < G; ++g) { mse[g] = 0.0f; qjl[g] = 0.0f; }
#pragma unroll 8
                for (int j = 0; j < D; ++j) {
                    const uint32_t code = (byte_at(kwv, 4 + j / 4) >> (2 * (j % 4))) & 3u;
                    const float c = sm.ktab[code];
                    const float sgn = ((byte_at(kwv, 4 + D / 4 + j / 8) >> (j % 8)) & 1u) ? 1.0f : -1.0f;
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        mse[g] = fmaf(sm.q[g * D + j], c, mse[g]);
                        qjl[g] = fmaf(sm.qs[g * D + j], sgn, qjl[g]);
                    }
                }
#pragma unroll
                for (int g = 0; g < G; ++g) t[g] = n * fmaf(gam, qjl[g], mse[g]);
            }

            // ---- 3. online softmax over the tile
            float* pw = sm.pw[w];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float tv = valid ? t[g] : -INFINITY;
                if (a.scores && valid)
                    a.scores[(static_cast<size_t>(b) * a.hq + hq0 + g) * a.capacity + t0 + lane] = tv * kLn2;
                const float mt = wave_max(tv);
                const float mn = fmaxf(m_run[g], mt);
                const float p = valid ? exp2f(tv - mn) : 0.0f;
                const float alpha = exp2f(m_run[g] - mn);  // 0 on the first tile (m_run = -inf)
                l_run[g] = l_run[g] * alpha + wave_sum(p);
                m_run[g] = mn;
#pragma unroll
                for (int k = 0; k < DPL; ++k) acc[g][k] *= alpha;
                pw[lane * G + g] = p;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

            // ---- 4. values, one lane per DPL coordinates
            const uint8_t* vt = sm.vtile[w];
            for (int i = 0; i < nv; ++i) {
                const uint8_t* vb = vt + i * VBV;
                float wgt[G];
#pragma unroll
                for (int g = 0; g < G; ++g) wgt[g] = pw[i * G + g];
                float val[DPL];
                if constexpr (VF == TQ_FMT_PQ4) {
                    constexpr int LPB = 128 / DPL;  // lanes per 128-block
                    const int blk = lane / LPB, lb = lane % LPB;
                    const uint8_t* bp = vb + 68 * blk;
                    const float n = half_bits_to_float(*reinterpret_cast<const uint16_t*>(bp));
                    if constexpr (DPL == 2) {
                        const float2 c = sm.vpair[bp[4 + lb]];
                        val[0] = n * c.x;
                        val[1] = n * c.y;
                    } else {
                        const uint32_t two = *reinterpret_cast<const uint16_t*>(bp + 4 + 2 * lb);
                        const float2 c0 = sm.vpair[two & 0xFFu], c1 = sm.vpair[two >> 8];
                        val[0] = n * c0.x; val[1] = n * c0.y; val[2] = n * c1.x; val[3] = n * c1.y;
                    }
                } else if constexpr (VF == TQ_FMT_PQ3) {
                    constexpr int LPB = 32 / DPL;
                    const int blk = lane / LPB, jb = DPL * (lane % LPB);
                    const uint8_t* bp = vb + 14 * blk;
                    const float n = half_bits_to_float(bp[0] | (bp[1] << 8));
                    const uint32_t lo = bp[2 + jb / 4] >> (2 * (jb % 4));
                    const uint32_t hi = bp[10 + jb / 8] >> (jb % 8);
#pragma unroll
                    for (int k = 0; k < DPL; ++k)
                        val[k] = n * sm.vtab[((lo >> (2 * k)) & 3u) | (((hi >> k) & 1u) << 2)];
                } else {  // GQ2V
                    constexpr int LPG = kGroup / DPL;
                    const int grp = lane / LPG, jb = DPL * (lane % LPG);
                    const uint8_t* gp = vb + 12 * grp;
                    const uint32_t sz = *reinterpret_cast<const uint32_t*>(gp);
                    const float sc = half_bits_to_float(sz & 0xFFFFu), zr = half_bits_to_float(sz >> 16);
                    const uint32_t q = gp[4 + jb / 4] >> (2 * (jb % 4));
#pragma unroll
                    for (int k = 0; k < DPL; ++k) val[k] = fmaf(static_cast<float>((q >> (2 * k)) & 3u), sc, zr);
                }
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int k = 0; k < DPL; ++k) acc[g][k] = fmaf(wgt[g], val[k], acc[g][k]);
            }
        }
        __syncthreads();  // tiles are overwritten on the next trip
    }

    // ---- merge the wavefronts of the workgroup and write the split record
    float* red = reinterpret_cast<float*>(&sm.ktile[0][0]);  // reuse: [kWaves][G][2 + D]
    static_assert(sizeof(sm.ktile) + sizeof(sm.vtile) >= sizeof(float) * kWaves * G * (2 + D), "merge buffer");
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float* r = red + (w * G + g) * (2 + D);
        if (lane == 0) { r[0] = m_run[g]; r[1] = l_run[g]; }
#pragma unroll
        for (int k = 0; k < DPL; ++k) r[2 + lane * DPL + k] = acc[g][k];
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += blockDim.x) {
        const int g = idx / D, j = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, red[(ww * G + g) * (2 + D)]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float* r = red + (ww * G + g) * (2 + D);
            const float f = r[0] == -INFINITY ? 0.0f : exp2f(r[0] - M);
            L = fmaf(r[1], f, L);
            A = fmaf(r[2 + j], f, A);
        }
        const size_t rec = rec0 + static_cast<size_t>(g) * a.splits;
        a.acc[rec * D + j] = A;
        if (j == 0) a.ml[rec] = make_float2(M, L);
    }
}

// ---------------------------------------------------------------------------
// Matrix-core variant for 4-bit PQ4 keys and values with G = 4 * NGRP query
// heads per KV head.  The two per-tile contractions
//     S[g][t] = sum_j q_rot[g][j] * c[code_tj]        (scores)
//     O[g][j] += sum_t w[g][t] * c[vcode_tj]          (values)
// have exactly four rows per head group, the shape of v_mfma_f32_4x4x1f32
// (16 independent 4x4 outer products, fp32 in and out).  The query is held
// with the A-broadcast layout: lane 4b+i of register r holds head i's
// coordinate 16r+b, and CBSZ=4/ABID=b broadcasts block b's four values to
// all blocks, so the rotated query of a head group costs d/16 registers and
// the 64 softmax weights of a tile 4 registers.  The VALU only unpacks
// codes, looks centroids up in an LDS pair table and runs the softmax.

constexpr int kPwStride = 80;  // floats per head row of the weight buffer (bank spread for the transposed read)
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int... I, typename F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

template <int D, int NGRP>
struct SmemMfma {
    static constexpr int VB = 68 * (D / 128);
    float ktab[16];                      // centroid of each 4-bit code (16 banks: lookups never conflict)
    float vtab[16];
    alignas(16) uint8_t ktile[kWaves][kTile * VB];
    alignas(16) uint8_t vtile[kWaves][kTile * VB];
    float pw[kWaves][4 * NGRP * kPwStride];  // w[h][t] of the current tile, padded rows
};

template <int D, int NGRP>
__global__ __launch_bounds__(kWaves * 64) void decode_partial_mfma_kernel(DecodeArgs a, DevCodebook cbk, DevCodebook cbv) {
    using SM = SmemMfma<D, NGRP>;
    constexpr int G = 4 * NGRP;
    constexpr int VB = SM::VB;
    constexpr int NB = D / 128;      // 68-byte blocks per vector
    constexpr int NR = D / 16;       // query registers per head group
    constexpr int DPL = D / 64;      // value coordinates per lane
    constexpr int CH = kTile * VB / 16;           // 16-byte chunks per tile
    constexpr int NCH = (CH + 63) / 64;           // chunks per lane
    __shared__ __align__(16) SM sm;

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int hq0 = h * G;
    int N = a.seq_lens[b];
    N = N < 0 ? 0 : (N > a.capacity ? a.capacity : N);
    const int start = s * a.split_len;
    const int end = min(start + a.split_len, N);
    const size_t rec0 = (static_cast<size_t>(b) * a.hq + hq0) * a.splits + s;

    if (start >= end) {
        for (int g = 0; g < G; ++g) {
            const size_t rec = rec0 + static_cast<size_t>(g) * a.splits;
            if (tid == 0) a.ml[rec] = make_float2(-INFINITY, 0.0f);
            for (int j = tid; j < D; j += blockDim.x) a.acc[rec * D + j] = 0.0f;
        }
        return;
    }

    if (tid < 16) {
        sm.ktab[tid] = cbk.centroids[tid];
        sm.vtab[tid] = cbv.centroids[tid];
    }

    // rotated query in the A-broadcast layout, scaled by log2(e)/sqrt(d)
    const float qscale = kLog2e / sqrtf(static_cast<float>(D));
    const int bl = lane >> 2, il = lane & 3;
    float qreg[NGRP][NR];
#pragma unroll
    for (int gr = 0; gr < NGRP; ++gr) {
        const float* qg = a.q_rot + (static_cast<size_t>(b) * a.hq + hq0 + 4 * gr + il) * D;
#pragma unroll
        for (int r = 0; r < NR; ++r) qreg[gr][r] = qg[16 * r + bl] * qscale;
    }
    __syncthreads();

    float m_run[G], l_run[G];
    f32x4 accv[NGRP][DPL];
#pragma unroll
    for (int g = 0; g < G; ++g) { m_run[g] = -INFINITY; l_run[g] = 0.0f; }
#pragma unroll
    for (int gr = 0; gr < NGRP; ++gr)
#pragma unroll
        for (int k = 0; k < DPL; ++k) accv[gr][k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const size_t stream_row = (static_cast<size_t>(b) * a.hkv + h) * a.capacity;
    const u32x4* kstream = reinterpret_cast<const u32x4*>(a.k_cache + stream_row * VB);
    const u32x4* vstream = reinterpret_cast<const u32x4*>(a.v_cache + stream_row * VB);
    u32x4* kd = reinterpret_cast<u32x4*>(sm.ktile[w]);
    u32x4* vd = reinterpret_cast<u32x4*>(sm.vtile[w]);
    float* pw = sm.pw[w];

    // register prefetch of the next tile (tiles are in bounds: t0 + 64 <= capacity)
    u32x4 kpre[NCH], vpre[NCH];
    int t0 = start + w * kTile;
    if (t0 < end) {
        const u32x4* ks = kstream + static_cast<size_t>(t0) * VB / 16;
        const u32x4* vs = vstream + static_cast<size_t>(t0) * VB / 16;
#pragma unroll
        for (int m = 0; m < NCH; ++m) {
            const int c = (lane + 64 * m) < CH ? lane + 64 * m : CH - 1;
            kpre[m] = ks[c];
            vpre[m] = vs[c];
        }
    }

    for (; t0 < end; t0 += kSplitQuantum) {
        const int nv = min(kTile, end - t0);
#pragma unroll
        for (int m = 0; m < NCH; ++m) {
            const int c = lane + 64 * m;
            if (c < CH) { kd[c] = kpre[m]; vd[c] = vpre[m]; }
        }
        if (t0 + kSplitQuantum < end) {
            const u32x4* ks = kstream + static_cast<size_t>(t0 + kSplitQuantum) * VB / 16;
            const u32x4* vs = vstream + static_cast<size_t>(t0 + kSplitQuantum) * VB / 16;
#pragma unroll
            for (int m = 0; m < NCH; ++m) {
                const int c = (lane + 64 * m) < CH ? lane + 64 * m : CH - 1;
                kpre[m] = ks[c];
                vpre[m] = vs[c];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- scores: lane = token, register i of group gr = head 4*gr+i
        const bool valid = lane < nv;
        f32x4 sc[NGRP];
#pragma unroll
        for (int gr = 0; gr < NGRP; ++gr) sc[gr] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const uint8_t* kb = sm.ktile[w] + lane * VB;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const uint32_t* kw = reinterpret_cast<const uint32_t*>(kb + 68 * blk);
            const float nk = half_bits_to_float(kw[0] & 0xFFFFu);
            f32x4 part[NGRP][2];
#pragma unroll
            for (int gr = 0; gr < NGRP; ++gr) part[gr][0] = part[gr][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                // nibble * 4 = byte offset into the 16-entry table: even codes
                // from (w << 2) & 0x3C.., odd codes from (w >> 2) & 0x3C..
                const uint32_t w0 = kw[1 + 2 * rr], w1 = kw[2 + 2 * rr];
                const uint32_t e0 = (w0 << 2) & 0x3C3C3C3Cu, o0 = (w0 >> 2) & 0x3C3C3C3Cu;
                const uint32_t e1 = (w1 << 2) & 0x3C3C3C3Cu, o1 = (w1 >> 2) & 0x3C3C3C3Cu;
                const char* kt = reinterpret_cast<const char*>(sm.ktab);
                float cv[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    cv[2 * q] = *reinterpret_cast<const float*>(kt + ((e0 >> (8 * q)) & 0xFFu));
                    cv[2 * q + 1] = *reinterpret_cast<const float*>(kt + ((o0 >> (8 * q)) & 0xFFu));
                    cv[8 + 2 * q] = *reinterpret_cast<const float*>(kt + ((e1 >> (8 * q)) & 0xFFu));
                    cv[8 + 2 * q + 1] = *reinterpret_cast<const float*>(kt + ((o1 >> (8 * q)) & 0xFFu));
                }
                const int r = 8 * blk + rr;
                static_for<16>([&](auto bc) {
                    constexpr int B = decltype(bc)::value;
                    const float val = cv[B];
#pragma unroll
                    for (int gr = 0; gr < NGRP; ++gr)
                        part[gr][rr & 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(qreg[gr][r], val, part[gr][rr & 1], 4, B, 0);
                });
            }
#pragma unroll
            for (int gr = 0; gr < NGRP; ++gr) sc[gr] += nk * (part[gr][0] + part[gr][1]);
        }

        // ---- online softmax per head; w = p * value norm to LDS, transposed
        const float nvn = half_bits_to_float(*reinterpret_cast<const uint16_t*>(sm.vtile[w] + lane * VB));
#pragma unroll
        for (int gr = 0; gr < NGRP; ++gr) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int g = 4 * gr + i;
                const float tv = valid ? sc[gr][i] : -INFINITY;
                if (a.scores && valid)
                    a.scores[(static_cast<size_t>(b) * a.hq + hq0 + g) * a.capacity + t0 + lane] = tv * kLn2;
                const float mt = wave_max(tv);
                const float mn = fmaxf(m_run[g], mt);
                const float p = valid ? exp2f(tv - mn) : 0.0f;
                const float alpha = exp2f(m_run[g] - mn);
                l_run[g] = fmaf(l_run[g], alpha, p);  // per-lane partial sum, reduced once per split
                m_run[g] = mn;
#pragma unroll
                for (int k = 0; k < DPL; ++k) accv[gr][k][i] *= alpha;
                pw[g * kPwStride + lane] = valid ? p * nvn : 0.0f;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float wreg[NGRP][4];
#pragma unroll
        for (int gr = 0; gr < NGRP; ++gr)
#pragma unroll
            for (int r = 0; r < 4; ++r) wreg[gr][r] = pw[(4 * gr + il) * kPwStride + 16 * r + bl];

        // ---- values: lane owns coordinates DPL*lane .. DPL*lane+DPL-1
        const int vblk = (DPL * lane) / 128;
        const int voff = 68 * vblk + 4 + ((DPL * lane) % 128) / 2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            static_for<16>([&](auto bc) {
                constexpr int B = decltype(bc)::value;
                const uint8_t* vb = sm.vtile[w] + (16 * r + B) * VB + voff;
                const char* vt = reinterpret_cast<const char*>(sm.vtab);
                float val[DPL];
                if constexpr (DPL == 2) {
                    const uint32_t by = vb[0];
                    val[0] = *reinterpret_cast<const float*>(vt + ((by << 2) & 0x3Cu));
                    val[1] = *reinterpret_cast<const float*>(vt + ((by >> 2) & 0x3Cu));
                } else {
                    const uint32_t two = *reinterpret_cast<const uint16_t*>(vb);
                    val[0] = *reinterpret_cast<const float*>(vt + ((two << 2) & 0x3Cu));
                    val[1] = *reinterpret_cast<const float*>(vt + ((two >> 2) & 0x3Cu));
                    val[2] = *reinterpret_cast<const float*>(vt + ((two >> 6) & 0x3Cu));
                    val[3] = *reinterpret_cast<const float*>(vt + ((two >> 10) & 0x3Cu));
                }
#pragma unroll
                for (int gr = 0; gr < NGRP; ++gr)
#pragma unroll
                    for (int k = 0; k < DPL; ++k)
                        accv[gr][k] = __builtin_amdgcn_mfma_f32_4x4x1f32(wreg[gr][r], val[k], accv[gr][k], 4, B, 0);
            });
        }
    }

    // ---- merge the wavefronts of the workgroup and write the split record
#pragma unroll
    for (int g = 0; g < G; ++g) l_run[g] = wave_sum(l_run[g]);
    __syncthreads();
    float* red = reinterpret_cast<float*>(&sm.ktile[0][0]);
    static_assert(sizeof(sm.ktile) + sizeof(sm.vtile) >= sizeof(float) * kWaves * G * (2 + D), "merge buffer");
#pragma unroll
    for (int gr = 0; gr < NGRP; ++gr)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = 4 * gr + i;
            float* r = red + (w * G + g) * (2 + D);
            if (lane == 0) { r[0] = m_run[g]; r[1] = l_run[g]; }
#pragma unroll
            for (int k = 0; k < DPL; ++k) r[2 + lane * DPL + k] = accv[gr][k][i];
        }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += blockDim.x) {
        const int g = idx / D, j = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, red[(ww * G + g) * (2 + D)]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float* r = red + (ww * G + g) * (2 + D);
            const float f = r[0] == -INFINITY ? 0.0f : exp2f(r[0] - M);
            L = fmaf(r[1], f, L);
            A = fmaf(r[2 + j], f, A);
        }
        const size_t rec = rec0 + static_cast<size_t>(g) * a.splits;
        a.acc[rec * D + j] = A;
        if (j == 0) a.ml[rec] = make_float2(M, L);
    }
}

// One workgroup per (b, query head): merge the split records, normalize and,
// for rotated value formats, rotate back once.  Each thread owns four
// coordinates of one split group, so the record rows stream in with 16-byte
// loads from many splits at once.
constexpr int kCombineThreads = 256;

template <int D, bool ROTATED>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(const float2* __restrict__ ml,
                                                                        const float* __restrict__ acc,
                                                                        float* __restrict__ out, int splits,
                                                                        DevCodebook cbv) {
    constexpr int TPR = D / 4;                    // threads per record row
    constexpr int NGS = kCombineThreads / TPR;    // split groups
    constexpr int DPL = D / 64;
    __shared__ float wave_m[kCombineThreads / 64];
    __shared__ float4 part[NGS][TPR];
    __shared__ float part_l[NGS];
    __shared__ float o_sh[D];
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const float2* mr = ml + static_cast<size_t>(row) * splits;
    float M = -INFINITY;
    for (int s = tid; s < splits; s += kCombineThreads) M = fmaxf(M, mr[s].x);
    M = wave_max(M);
    if (lane == 0) wave_m[tid >> 6] = M;
    __syncthreads();
    M = fmaxf(fmaxf(wave_m[0], wave_m[1]), fmaxf(wave_m[2], wave_m[3]));
    const int grp = tid / TPR, c = tid % TPR;
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float L = 0.0f;
    if (M != -INFINITY) {
        const float4* ar = reinterpret_cast<const float4*>(acc) + static_cast<size_t>(row) * splits * TPR + c;
#pragma unroll 4
        for (int s = grp; s < splits; s += NGS) {
            const float2 r = mr[s];
            const float f = r.x == -INFINITY ? 0.0f : exp2f(r.x - M);
            const float4 v = ar[static_cast<size_t>(s) * TPR];
            L = fmaf(r.y, f, L);
            o.x = fmaf(v.x, f, o.x); o.y = fmaf(v.y, f, o.y); o.z = fmaf(v.z, f, o.z); o.w = fmaf(v.w, f, o.w);
        }
    }
    part[grp][c] = o;
    if (c == 0) part_l[grp] = L;
    __syncthreads();
    if (tid < TPR) {
        float4 t = part[0][tid];
        float Lt = part_l[0];
#pragma unroll
        for (int g = 1; g < NGS; ++g) {
            const float4 u = part[g][tid];
            t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
            Lt += part_l[g];
        }
        const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
        o_sh[4 * tid] = t.x * inv;
        o_sh[4 * tid + 1] = t.y * inv;
        o_sh[4 * tid + 2] = t.z * inv;
        o_sh[4 * tid + 3] = t.w * inv;
    }
    __syncthreads();
    if (tid >= 64) return;
    float v[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) v[k] = o_sh[DPL * lane + k];
    if constexpr (ROTATED) {
        // o <- Pi^T o = diag(s) H o / sqrt(d); element j = DPL*lane + k
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
        constexpr float kInvSqrtD = D == 256 ? 0.0625f : 0.08838834764831845f;
#pragma unroll
        for (int k = 0; k < DPL; ++k) v[k] *= kInvSqrtD * rotation_sign(cbv, DPL * lane + k);
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) out[static_cast<size_t>(row) * D + DPL * lane + k] = v[k];
}

int auto_split_tokens(const tq_layout* L) {
    const long streams = static_cast<long>(L->batch) * L->n_kv_heads;
    const long max_splits = (L->capacity + kSplitQuantum - 1) / kSplitQuantum;
    long want = (4096 + streams - 1) / streams;  // aim at >= 4096 workgroups
    if (want > max_splits) want = max_splits;
    if (want < 1) want = 1;
    long len = (L->capacity + want - 1) / want;
    len = (len + kSplitQuantum - 1) / kSplitQuantum * kSplitQuantum;
    return static_cast<int>(len);
}

int resolve_splits(const tq_layout* L, int split_tokens, int* split_len) {
    if (split_tokens < 0 || split_tokens % kSplitQuantum) return 0;
    const int len = split_tokens == 0 ? auto_split_tokens(L) : split_tokens;
    *split_len = len;
    return (L->capacity + len - 1) / len;
}

template <int KF, int VF, int D, int G>
int launch_partial(const DecodeArgs& a, const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv,
                   hipStream_t st) {
    dim3 grid(a.splits, L->n_kv_heads, L->batch);
    hipLaunchKernelGGL((decode_partial_kernel<KF, VF, D, G>), grid, dim3(kWaves * 64), 0, st, a, to_dev(cbk),
                       to_dev(cbv));
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

template <int D, int NGRP>
int launch_partial_mfma(const DecodeArgs& a, const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv,
                        hipStream_t st) {
    dim3 grid(a.splits, L->n_kv_heads, L->batch);
    hipLaunchKernelGGL((decode_partial_mfma_kernel<D, NGRP>), grid, dim3(kWaves * 64), 0, st, a, to_dev(cbk),
                       to_dev(cbv));
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

template <int KF, int VF, int D>
int dispatch_group(int G, const DecodeArgs& a, const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv,
                   hipStream_t st) {
    if constexpr (KF == TQ_FMT_PQ4 && VF == TQ_FMT_PQ4) {
        if (G == 4) return launch_partial_mfma<D, 1>(a, L, cbk, cbv, st);
        if (G == 8) return launch_partial_mfma<D, 2>(a, L, cbk, cbv, st);
    }
    switch (G) {
        case 1: return launch_partial<KF, VF, D, 1>(a, L, cbk, cbv, st);
        case 2: return launch_partial<KF, VF, D, 2>(a, L, cbk, cbv, st);
        case 4: return launch_partial<KF, VF, D, 4>(a, L, cbk, cbv, st);
        case 5: return launch_partial<KF, VF, D, 5>(a, L, cbk, cbv, st);
        case 8: return launch_partial<KF, VF, D, 8>(a, L, cbk, cbv, st);
        default: return TQ_ERR_UNSUPPORTED;
    }
}

template <int KF, int VF>
int dispatch_dim(const DecodeArgs& a, const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv,
                 hipStream_t st) {
    const int G = L->n_q_heads / L->n_kv_heads;
    return L->head_dim == 128 ? dispatch_group<KF, VF, 128>(G, a, L, cbk, cbv, st)
                              : dispatch_group<KF, VF, 256>(G, a, L, cbk, cbv, st);
}

int check_decode(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv) {
    int st = check_layout(L);
    if (st != TQ_OK) return st;
    if ((st = check_codebook(cbk, L->k_format, L->head_dim)) != TQ_OK) return st;
    if ((st = check_codebook(cbv, L->v_format, L->head_dim)) != TQ_OK) return st;
    const int G = L->n_q_heads / L->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 5 && G != 8) return TQ_ERR_UNSUPPORTED;
    return TQ_OK;
}

}  // namespace
}  // namespace tq

extern "C" {

int tq_decode_splits(const tq_layout* L, int split_tokens) {
    if (tq::check_layout(L) != TQ_OK) return 0;
    int len = 0;
    return tq::resolve_splits(L, split_tokens, &len);
}

size_t tq_decode_workspace_bytes(const tq_layout* L, int split_tokens) {
    const int splits = tq_decode_splits(L, split_tokens);
    if (splits <= 0) return 0;
    const size_t recs = static_cast<size_t>(L->batch) * L->n_q_heads * splits;
    return recs * sizeof(float2) + recs * L->head_dim * sizeof(float);
}

int tq_decode_partial(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const float* q_rot,
                      const float* q_sketch, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                      float* scores, int split_tokens, void* ws, size_t ws_bytes, hipStream_t stream) {
    using namespace tq;
    int st = check_decode(L, cbk, cbv);
    if (st != TQ_OK) return st;
    int len = 0;
    const int splits = resolve_splits(L, split_tokens, &len);
    if (splits <= 0) return TQ_ERR_INVALID;
    if (!q_rot || !k_cache || !v_cache || !seq_lens || !ws) return TQ_ERR_INVALID;
    if (L->k_format == TQ_FMT_TQ3K && !q_sketch) return TQ_ERR_INVALID;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(ws, 16) || !aligned(q_rot, 4) ||
        !aligned(seq_lens, 4) || (scores && !aligned(scores, 4)) || (q_sketch && !aligned(q_sketch, 4)))
        return TQ_ERR_INVALID;
    if (ws_bytes < tq_decode_workspace_bytes(L, split_tokens)) return TQ_ERR_WORKSPACE;
    DecodeArgs a{};
    a.q_rot = q_rot;
    a.q_sk = q_sketch;
    a.k_cache = static_cast<const uint8_t*>(k_cache);
    a.v_cache = static_cast<const uint8_t*>(v_cache);
    a.seq_lens = seq_lens;
    a.scores = scores;
    const size_t recs = static_cast<size_t>(L->batch) * L->n_q_heads * splits;
    a.ml = static_cast<float2*>(ws);
    a.acc = reinterpret_cast<float*>(static_cast<char*>(ws) + recs * sizeof(float2));
    a.hq = L->n_q_heads;
    a.hkv = L->n_kv_heads;
    a.capacity = L->capacity;
    a.splits = splits;
    a.split_len = len;
    const int kf = L->k_format, vf = L->v_format;
    if (kf == TQ_FMT_PQ4 && vf == TQ_FMT_PQ4) return dispatch_dim<TQ_FMT_PQ4, TQ_FMT_PQ4>(a, L, *cbk, *cbv, stream);
    if (kf == TQ_FMT_PQ3 && vf == TQ_FMT_PQ3) return dispatch_dim<TQ_FMT_PQ3, TQ_FMT_PQ3>(a, L, *cbk, *cbv, stream);
    if (kf == TQ_FMT_PQ3 && vf == TQ_FMT_PQ4) return dispatch_dim<TQ_FMT_PQ3, TQ_FMT_PQ4>(a, L, *cbk, *cbv, stream);
    if (kf == TQ_FMT_TQ3K && vf == TQ_FMT_GQ2V) return dispatch_dim<TQ_FMT_TQ3K, TQ_FMT_GQ2V>(a, L, *cbk, *cbv, stream);
    return TQ_ERR_UNSUPPORTED;
}

int tq_decode_combine(const tq_layout* L, const tq_codebook* cbv, int split_tokens, const void* ws, size_t ws_bytes,
                      float* out, hipStream_t stream) {
    using namespace tq;
    int st = check_layout(L);
    if (st != TQ_OK) return st;
    if ((st = check_codebook(cbv, L->v_format, L->head_dim)) != TQ_OK) return st;
    int len = 0;
    const int splits = resolve_splits(L, split_tokens, &len);
    if (splits <= 0 || !ws || !out || !aligned(ws, 16) || !aligned(out, 4)) return TQ_ERR_INVALID;
    if (ws_bytes < tq_decode_workspace_bytes(L, split_tokens)) return TQ_ERR_WORKSPACE;
    const size_t recs = static_cast<size_t>(L->batch) * L->n_q_heads * splits;
    const float2* ml = static_cast<const float2*>(ws);
    const float* acc = reinterpret_cast<const float*>(static_cast<const char*>(ws) + recs * sizeof(float2));
    const int rows = L->batch * L->n_q_heads;
    const bool rot = L->v_format != TQ_FMT_GQ2V;
    const DevCodebook c = to_dev(*cbv);
    if (L->head_dim == 128) {
        if (rot) hipLaunchKernelGGL((decode_combine_kernel<128, true>), dim3(rows), dim3(kCombineThreads), 0, stream, ml, acc, out, splits, c);
        else hipLaunchKernelGGL((decode_combine_kernel<128, false>), dim3(rows), dim3(kCombineThreads), 0, stream, ml, acc, out, splits, c);
    } else {
        if (rot) hipLaunchKernelGGL((decode_combine_kernel<256, true>), dim3(rows), dim3(kCombineThreads), 0, stream, ml, acc, out, splits, c);
        else hipLaunchKernelGGL((decode_combine_kernel<256, false>), dim3(rows), dim3(kCombineThreads), 0, stream, ml, acc, out, splits, c);
    }
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

int tq_decode_attention(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const float* q_rot,
                        const float* q_sketch, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                        float* out, float* scores, int split_tokens, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!out) return TQ_ERR_INVALID;
    int st = tq_decode_partial(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, seq_lens, scores, split_tokens, ws,
                               ws_bytes, stream);
    if (st != TQ_OK) return st;
    return tq_decode_combine(L, cbv, split_tokens, ws, ws_bytes, out, stream);
}

}  // extern "C"
