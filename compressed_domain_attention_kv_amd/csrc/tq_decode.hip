// Read path of libtq on gfx950: the split-K partial of fused decode attention
// over compressed KV, and the C entry points of the decode.
//
// Each (batch row, KV head) stream is cut into context splits; a split
// record (m, l, acc) per query head holds its online-softmax state, with
// scores in log2 units and acc in the values' rotated basis.  Three kernels:
//   * decode_partial_sparse_kernel (PQ4 keys and values, d 128, G 4 or 8):
//     both contractions on the 2:4-sparse bf16 matrix instruction, centroids
//     from a replicated byte-pair table in LDS;
//   * decode_partial_bf16_kernel (PQ4 at d 256, and G 8 with distinct key
//     and value centroids): dense bf16 matrix products with nibble tables;
//   * decode_partial_kernel (every format pair and G): one lane per token for
//     scores, one lane per d/64 coordinates for values, on the VALU.
// The merge of the records (and the ring part of the hybrid read) lives in
// tq_combine.hip.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <utility>

#include "tq_device.h"
#include "tq_pq4.h"

namespace tq {
namespace {

constexpr float kLn2 = 0.6931471805599453f;

template <int FMT, int D>
constexpr int vbytes() {
    return FMT == TQ_FMT_PQ4 ? 68 * (D / 128)
         : FMT == TQ_FMT_PQ3 ? 14 * (D / 32)
         : FMT == TQ_FMT_TQ3K ? 4 + D / 4 + D / 8
         : FMT == TQ_FMT_GQ2V ? 12 * (D / kGroup)
                              : 20 * (D / kGroup);
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
    // Sparse V: a token whose weight against the running maximum, e^(s - m), is below
    // v_skip adds nothing to the value sum (its weight still enters the denominator), and
    // value work is skipped where no weight survives.  0 keeps every value.
    float v_skip;
    // the unrotated query [B][Hq][D], when the kernel rotates it itself (q_rot unused)
    const float* q_raw;
    // the step's new token, when the kernel appends it itself: fp16 rows [B][Hkv][D] of K
    // and V, written at position new_pos[b] of each stream (skipped when outside the cache)
    const uint16_t* k_new;
    const uint16_t* v_new;
    const int32_t* new_pos;
    uint8_t* k_wr;
    uint8_t* v_wr;
    // when out is set, the workgroup that finishes a stream last merges the stream's split
    // records into the attention output (fp32 [B][Hq][D]); arrivals[b * hkv + h] counts the
    // stream's finished workgroups and is zero before and after the launch
    float* out;
    uint32_t* arrivals;
};

// byte k of a register-resident little-endian byte run (k known at compile time after unrolling)
template <int N>
__device__ __forceinline__ uint32_t byte_at(const uint32_t (&w)[N], int k) {
    return (w[k >> 2] >> (8 * (k & 3))) & 0xFFu;
}

// 16 bytes of a cache stream, read with the non-temporal policy (each byte is read
// once per decode; streaming reads measured faster with it)
__device__ __forceinline__ uint4 stream_load16(const uint4* p) {
    typedef uint32_t v4 __attribute__((ext_vector_type(4)));
    const v4 x = __builtin_nontemporal_load(reinterpret_cast<const v4*>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
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

// Merge of the per-wavefront partials of a workgroup, red[w][head][2 + D] = (m, l, acc[D]) in
// log2 units, into one split record per head ([P2] trick 3: the running (m, l, acc) states
// combine by rescaling to the common maximum).  Threads 0 .. G-1 take, per head, the maximum
// M, the factors 2^(m_w - M) (0 for a wavefront without tokens) into fw[w][head] and the
// record's (M, sum_w l_w f_w); after a barrier every coordinate is sum_w f_w acc_w, the sums
// in wavefront order.
template <int D, int G, int NWV>
__device__ __forceinline__ void merge_factors(const float* red, float* fw, int t, float2* ml, int splits) {
    if (t < G) {
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NWV; ++ww) M = fmaxf(M, red[(ww * G + t) * (2 + D)]);
        float L = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NWV; ++ww) {
            const float* r = red + (ww * G + t) * (2 + D);
            const float f = r[0] == -INFINITY ? 0.0f : exp2f(r[0] - M);
            fw[ww * G + t] = f;
            L = fmaf(r[1], f, L);
        }
        ml[static_cast<size_t>(t) * splits] = make_float2(M, L);
    }
}
template <int D, int G, int NWV>
__device__ __forceinline__ float merged_coordinate(const float* red, const float* fw, int gg, int j) {
    float A = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) A = fmaf(red[(ww * G + gg) * (2 + D) + 2 + j], fw[ww * G + gg], A);
    return A;
}

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
            for (int c = lane; c < CK; c += 64) kd[c] = stream_load16(ks + c);
#pragma unroll
            for (int c = lane; c < CV; c += 64) vd[c] = stream_load16(vs + c);
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
                pw[lane * G + g] = p >= a.v_skip ? p : 0.0f;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

            // ---- 4. values, one lane per DPL coordinates
            const uint8_t* vt = sm.vtile[w];
            for (int i = 0; i < nv; ++i) {
                const uint8_t* vb = vt + i * VBV;
                float wgt[G];
                bool keep = false;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    wgt[g] = pw[i * G + g];
                    keep = keep || wgt[g] != 0.0f;
                }
                if (!keep) continue;  // the same for every lane: no value to decode
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
                } else if constexpr (VF == TQ_FMT_GQ2V) {
                    constexpr int LPG = kGroup / DPL;
                    const int grp = lane / LPG, jb = DPL * (lane % LPG);
                    const uint8_t* gp = vb + 12 * grp;
                    const uint32_t sz = *reinterpret_cast<const uint32_t*>(gp);
                    const float sc = half_bits_to_float(sz & 0xFFFFu), zr = half_bits_to_float(sz >> 16);
                    const uint32_t q = gp[4 + jb / 4] >> (2 * (jb % 4));
#pragma unroll
                    for (int k = 0; k < DPL; ++k) val[k] = fmaf(static_cast<float>((q >> (2 * k)) & 3u), sc, zr);
                } else {  // GQ4V: nibble codes, channel j of a group in byte j/2
                    constexpr int LPG = kGroup / DPL;
                    const int grp = lane / LPG, jb = DPL * (lane % LPG);
                    const uint8_t* gp = vb + 20 * grp;
                    const uint32_t sz = *reinterpret_cast<const uint32_t*>(gp);
                    const float sc = half_bits_to_float(sz & 0xFFFFu), zr = half_bits_to_float(sz >> 16);
                    // DPL nibbles from byte jb / 2 on (jb is a multiple of DPL: aligned reads)
                    const uint32_t q = DPL == 2 ? gp[4 + jb / 2] : *reinterpret_cast<const uint16_t*>(gp + 4 + jb / 2);
#pragma unroll
                    for (int k = 0; k < DPL; ++k) val[k] = fmaf(static_cast<float>((q >> (4 * k)) & 15u), sc, zr);
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
    __shared__ float fw[kWaves * G];
    merge_factors<D, G, kWaves>(red, fw, tid, a.ml + rec0, a.splits);
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += blockDim.x) {
        const int g = idx / D, j = idx % D;
        const size_t rec = rec0 + static_cast<size_t>(g) * a.splits;
        a.acc[rec * D + j] = merged_coordinate<D, G, kWaves>(red, fw, g, j);
    }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));


// Byte offset into a 32-entry table from byte Q of a pre-shifted code word:
// (byte_Q(x) & 0x7C), one sub-dword (SDWA) VALU operation.  The result only
// ever feeds an LDS address.
#define TQ_NIBBLE_OFFSET(Q)                                                                              \
    template <>                                                                                          \
    __device__ __forceinline__ uint32_t nibble_offset<Q>(uint32_t x) {                                   \
        uint32_t r;                                                                                      \
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_" #Q \
            : "=v"(r) : "v"(0x7Cu), "v"(x));                                                             \
        return r;                                                                                        \
    }
template <int Q>
__device__ __forceinline__ uint32_t nibble_offset(uint32_t x);
TQ_NIBBLE_OFFSET(0)
TQ_NIBBLE_OFFSET(1)
TQ_NIBBLE_OFFSET(2)
TQ_NIBBLE_OFFSET(3)
#undef TQ_NIBBLE_OFFSET

// The eight table entries of a dword of PQ4 codes (coordinate 2q = low
// nibble of byte q) from two 32-entry tables, lo[k] = T[k & 15] and
// hi[k] = T[k >> 1]: with xl = w << 2, byte q of xl masked by 0x7C is
// (byte_q & 31) * 4; with xh = w >> 1 it is (byte_q >> 3) * 4.  A 32-entry
// table of words occupies each of the 32 LDS banks once, so the 64 lanes'
// lookups never conflict.
template <typename E>
__device__ __forceinline__ void decode_word(uint32_t w, const char* lo, const char* hi, E (&c)[8]) {
    const uint32_t xl = w << 2, xh = w >> 1;
    static_for<4>([&](auto qc) {
        constexpr int Q = decltype(qc)::value;
        c[2 * Q] = *reinterpret_cast<const E*>(lo + nibble_offset<Q>(xl));
        c[2 * Q + 1] = *reinterpret_cast<const E*>(hi + nibble_offset<Q>(xh));
    });
}

// Table entries of nibbles 4H..4H+3 of a code word, given xl = w << 2 and
// xh = w >> 1 (the same tables and masks as decode_word).
template <int H>
__device__ __forceinline__ void decode_half(uint32_t xl, uint32_t xh, const char* lo, const char* hi, uint32_t (&c)[4]) {
    c[0] = *reinterpret_cast<const uint32_t*>(lo + nibble_offset<2 * H>(xl));
    c[1] = *reinterpret_cast<const uint32_t*>(hi + nibble_offset<2 * H>(xh));
    c[2] = *reinterpret_cast<const uint32_t*>(lo + nibble_offset<2 * H + 1>(xl));
    c[3] = *reinterpret_cast<const uint32_t*>(hi + nibble_offset<2 * H + 1>(xh));
}

// Program-order point between phases that touch the same LDS bytes through
// differently typed accesses (no instruction is emitted).
// Workgroup barrier for LDS data written by the wavefronts themselves (ds writes), which
// leaves buffer loads in flight: a __syncthreads() would also wait for every buffer-to-LDS
// load still pending.  A stage filled by such loads is read only after the reading
// wavefront's own wait for them.
__device__ __forceinline__ void lds_write_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// An LDS word or byte offset that the optimizer keeps whole.  The LDS lowering gives
// an access an alias scope only when its address lies a few steps below the LDS
// variable; an access built from more steps goes unscoped, and the compiler then
// makes it wait for every buffer-to-LDS load still in flight (this tile's value
// stage included).  Addresses written as array + lds_offset(o) (+ a constant) stay
// shallow.  ON = false passes o through (kernels without buffer-to-LDS loads).
template <bool ON = true>
__device__ __forceinline__ uint32_t lds_offset(uint32_t o) {
    if constexpr (ON) asm("" : "+v"(o));
    return o;
}

// Online-softmax rescale threshold (log2 units): the running reference m is
// moved to the maximum only when some score exceeds m + kRescaleSlack, so
// weights 2^(s - m) stay below 2^kRescaleSlack and a tile without a new
// maximum costs one compare-and-ballot.  Any reference gives the same
// softmax; only overflow has to be excluded.
constexpr float kRescaleSlack = 8.0f;

// MFMA jobs whose centroid lookups are in flight ahead of the product that
// consumes the oldest (four lookups each; lgkmcnt counts at most 15).
constexpr int kLookahead = 3;

// bf16 bits nearest to a finite float
__device__ __forceinline__ uint32_t bf16_rn(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi), packed as (lo << 16) | hi
__device__ __forceinline__ uint32_t bf16_split(float x) {
    const uint32_t h = bf16_rn(x);
    return (bf16_rn(x - __uint_as_float(h << 16)) << 16) | h;
}
// the upper 16 bits of x in both halves
__device__ __forceinline__ uint32_t dup_hi16(uint32_t x) { return __builtin_amdgcn_perm(x, x, 0x03020302u); }

// Sum / maximum over each row of 16 lanes, the result in every lane of the row.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppHalfMirror>(x);
    x += dpp<kDppMirror>(x);
    return x;
}
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp<kDppXor1>(x));
    x = fmaxf(x, dpp<kDppXor2>(x));
    x = fmaxf(x, dpp<kDppHalfMirror>(x));
    x = fmaxf(x, dpp<kDppMirror>(x));
    return x;
}

// ---------------------------------------------------------------------------
// Merge of a stream's split records inside the decode launch ([P2] trick 3: the
// (m, l, acc) state of the splits is combined once, and acc / l taken once, at the
// end).  Each XCD has an L2 of its own, so the records are written with device-scope
// stores (write-through past the L2) and read back with device-scope loads; a
// workgroup waits for its own stores to complete, then counts itself in
// arrivals[b * hkv + h] with a device-scope atomic.  The workgroup that arrives last
// (it has seen every other increment, each issued after that workgroup's stores had
// completed) merges the G rows of the stream with the arithmetic of the combine
// kernel, normalizes, rotates back once (rotated value formats) and writes the
// output; it then sets the counter back to zero for the next launch.  No workgroup
// waits for another, and no L2 is written back or invalidated.

__device__ __forceinline__ void store_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(float2* p, float2 v) {
    const uint64_t bits = (static_cast<uint64_t>(__float_as_uint(v.y)) << 32) | __float_as_uint(v.x);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_dev(const float2* p) {
    const uint64_t bits =
        __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float2*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float(static_cast<uint32_t>(bits)), __uint_as_float(static_cast<uint32_t>(bits >> 32)));
}

// Workgroup-wide; true in the workgroup that finished stream (b, h) last.  flag_sh is
// one LDS word.  Every record store of the workgroup precedes the call.
__device__ __forceinline__ bool stream_arrive(const DecodeArgs& a, int b, int h, uint32_t* flag_sh) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's record stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(a.arrivals + (static_cast<size_t>(b) * a.hkv + h), 1u,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag_sh = prev + 1 == gridDim.x ? 1u : 0u;
    }
    __syncthreads();
    return *flag_sh != 0;
}

// The last workgroup's merge of rows hq0 .. hq0 + G - 1 with NT threads: NT / G
// threads per row, each owning four coordinates of one of its row's split groups and
// merging that group's records with a running maximum of its own, in batches of four
// records whose loads are all issued first; then the groups merge through LDS, and
// wavefront r rotates row r back and normalizes it.  With 256 threads per row this
// is exactly the combine kernel's order of operations.  lds: 4 NT + (2 NGS + D + 1) G
// floats.
template <int D, int G, int NT>
__device__ __forceinline__ void stream_merge(const DecodeArgs& a, const DevCodebook& cbv, bool rotated, int b, int hq0,
                                             float* lds) {
    constexpr int TPR = NT / G, C = D / 4, NGS = TPR / C, DPL = D / 64, SPT = 4;
    static_assert(NT % G == 0 && TPR % C == 0 && NGS >= 1, "whole split groups per row");
    static_assert(NT / 64 >= G, "a wavefront per row for the rotation back");
    constexpr float kInvSqrtD = D == 256 ? 0.0625f : 0.08838834764831845f;
    float4* part = reinterpret_cast<float4*>(lds);
    float* pm = lds + 4 * NT;
    float* pl = pm + G * NGS;
    float* fin = pl + G * NGS;
    float* finl = fin + G * D;
    const int tid = threadIdx.x, r = tid / TPR, u = tid % TPR, grp = u / C, c = u % C;
    const size_t row = static_cast<size_t>(b) * a.hq + hq0 + r;
    const float2* mr = a.ml + row * a.splits;
    const float4* ar = reinterpret_cast<const float4*>(a.acc) + row * a.splits * C + c;
    float Mt = -INFINITY, Lt = 0.0f;
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int s0 = grp; s0 < a.splits; s0 += SPT * NGS) {
        float2 rc[SPT];
        float4 v[SPT];
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            const int s = min(s0 + k * NGS, a.splits - 1);
            rc[k] = load_dev(mr + s);
            const float* x = reinterpret_cast<const float*>(ar + static_cast<size_t>(s) * C);
            v[k] = make_float4(load_dev(x), load_dev(x + 1), load_dev(x + 2), load_dev(x + 3));
        }
        float mb = Mt;
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            if (s0 + k * NGS >= a.splits) rc[k].x = -INFINITY;  // the reread past the last split weighs nothing
            mb = fmaxf(mb, rc[k].x);
        }
        const bool none = mb == -INFINITY;
        const float so = none ? 1.0f : exp2f(Mt - mb);
        Lt *= so;
        o.x *= so; o.y *= so; o.z *= so; o.w *= so;
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            const float f = rc[k].x == -INFINITY ? 0.0f : exp2f(rc[k].x - mb);
            Lt = fmaf(rc[k].y, f, Lt);
            o.x = fmaf(v[k].x, f, o.x); o.y = fmaf(v[k].y, f, o.y);
            o.z = fmaf(v[k].z, f, o.z); o.w = fmaf(v[k].w, f, o.w);
        }
        Mt = mb;
    }
    part[tid] = o;
    if (c == 0) {
        pm[r * NGS + grp] = Mt;
        pl[r * NGS + grp] = Lt;
    }
    __syncthreads();
    if (tid < G * C) {
        const int rr = tid / C, cc = tid % C;
        float M = pm[rr * NGS];
#pragma unroll
        for (int g = 1; g < NGS; ++g) M = fmaxf(M, pm[rr * NGS + g]);
        float4 t = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float L = 0.0f;
        if (M != -INFINITY) {
#pragma unroll
            for (int g = 0; g < NGS; ++g) {
                const float f = exp2f(pm[rr * NGS + g] - M);
                const float4 x = part[rr * TPR + g * C + cc];
                t.x = fmaf(x.x, f, t.x); t.y = fmaf(x.y, f, t.y);
                t.z = fmaf(x.z, f, t.z); t.w = fmaf(x.w, f, t.w);
                L = fmaf(pl[rr * NGS + g], f, L);
            }
        }
        *reinterpret_cast<float4*>(fin + rr * D + 4 * cc) = t;
        if (cc == 0) finl[rr] = L;
    }
    __syncthreads();
    const int wv = tid >> 6, lane = tid & 63;
    if (wv < G) {
        float v[DPL];
#pragma unroll
        for (int k = 0; k < DPL; ++k) v[k] = fin[wv * D + DPL * lane + k];
        if (rotated) {  // o <- Pi^T o = diag(s) H o / sqrt(d)
            wht_wave<DPL>(v, lane);
#pragma unroll
            for (int k = 0; k < DPL; ++k) v[k] *= kInvSqrtD * rotation_sign(cbv, DPL * lane + k);
        }
        const float L = finl[wv];
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
        for (int k = 0; k < DPL; ++k)
            a.out[(static_cast<size_t>(b) * a.hq + hq0 + wv) * D + DPL * lane + k] = v[k] * inv;
    }
}

// The end of a decode workgroup: when the launch merges, arrive, and merge the stream
// if this workgroup is its last.  Uniform over the workgroup.
template <int D, int G, int NT>
__device__ __forceinline__ void stream_finish(const DecodeArgs& a, const DevCodebook& cbv, bool rotated, int b, int h,
                                              float* lds, uint32_t* flag_sh) {
    if (a.out == nullptr) return;
    if (!stream_arrive(a, b, h, flag_sh)) return;
    stream_merge<D, G, NT>(a, cbv, rotated, b, h * G, lds);
    if (threadIdx.x == 0)
        __hip_atomic_store(a.arrivals + (static_cast<size_t>(b) * a.hkv + h), 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int G, int TT>
struct Bf16Cfg {
    static constexpr int VB = 68 * (D / 128);     // bytes per token and tensor
    static constexpr int NB = D / 128;            // 68-byte blocks per vector
    static constexpr int NTB = TT / 16;           // 16-token blocks per tile
    static constexpr int ROWS = 2 * G;            // MFMA rows in use: (head, hi/lo)
    static constexpr int WA = NB * NTB * ROWS * 16 + (ROWS < 16 ? 16 : 0);  // weight words per wavefront (+ zero row)
};

template <int D, int G, int TT>
struct SmemBf16 {
    using C = Bf16Cfg<D, G, TT>;
    uint32_t klo[32], khi[32], vlo[32], vhi[32];  // centroid pairs: lo[k] = P[k & 15], hi[k] = P[k >> 1]
    union {
        struct {
            alignas(16) uint32_t wa[kWaves][C::WA];  // value-product A operand [blk][tb][row][token] (+ zero row)
            alignas(16) u32x4 qa[8 * C::NB][64];     // score A operand per chunk and lane (shared by the wavefronts)
        } op;
        float red[kWaves * G * (2 + D)];            // per-wavefront (m, l, acc) records after the tile loop
    } u;
};

typedef uint32_t u32x4u __attribute__((ext_vector_type(4), aligned(4)));  // 16 bytes at a 4-byte boundary

// Key bytes of one tile as the score products consume them: lane (n, g)
// holds, for token 16 tb + n, the fp16 block norm and code words 4g..4g+3
// (coordinates 32g..32g+31) of every 68-byte block.
template <int NTB, int NB>
struct KeyTile {
    u32x4u w[NTB][NB];
    uint16_t norm[NTB][NB];
};
// Value bytes of one tile: lane (n, g) holds code word n of tokens
// 16 tb + 4g + u (u = 0..3) and the fp16 norm of token 16 tb + n.
template <int NTB, int NB>
struct ValueTile {
    uint32_t w[NTB][NB][4];
    uint16_t norm[NTB][NB];
};

// Raw buffer view of one cache stream: loads take a per-lane byte offset
// fixed for the whole split plus a wave-uniform tile offset in an SGPR, so
// a tile's loads cost no address arithmetic.  Only whole tiles inside the
// stream are requested through it (the SGPR offset is not range-checked).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const uint8_t* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                             0x00020000);
}

// Cache policy of the cache-stream loads: nt (non-temporal).  Every cache byte is read
// once per decode, and streaming reads with nt measured about 7% more bandwidth on
// MI355X than default-policy reads (6.7 vs 6.1 TB/s median over 570 MB).
constexpr int kStreamPolicy = 2;

// A resource of zero bytes: loads through it return zeros and read no memory.  The
// request for "the next tile" after a wavefront's last tile goes through it, so the
// loads stay unconditional (one path for the compiler's waits) at no HBM cost.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t null_rsrc(const uint8_t* base) { return stream_rsrc(base, 0); }

template <int VB, int NTB, int NB>
__device__ __forceinline__ void load_keys(KeyTile<NTB, NB>& k, __amdgpu_buffer_rsrc_t r, int norm_off, int word_off,
                                          int tile_off) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const int o = (16 * tb) * VB + 68 * blk;
            k.norm[tb][blk] = __builtin_amdgcn_raw_buffer_load_b16(r, norm_off + o, tile_off, kStreamPolicy);
            k.w[tb][blk] = __builtin_bit_cast(u32x4u, __builtin_amdgcn_raw_buffer_load_b128(r, word_off + o, tile_off,
                                                                                          kStreamPolicy));
        }
}
template <int VB, int NTB, int NB>
__device__ __forceinline__ void load_values(ValueTile<NTB, NB>& v, __amdgpu_buffer_rsrc_t r, int norm_off, int word_off,
                                            int tile_off) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            v.norm[tb][blk] = __builtin_amdgcn_raw_buffer_load_b16(r, norm_off + (16 * tb) * VB + 68 * blk, tile_off,
                                                                   kStreamPolicy);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v.w[tb][blk][u] = __builtin_amdgcn_raw_buffer_load_b32(r, word_off + (16 * tb + u) * VB + 68 * blk,
                                                                       tile_off, kStreamPolicy);
        }
}

// A wavefront's value tile of BYTES bytes, HBM -> LDS by buffer loads with an LDS
// destination: whole kilobytes with 16 bytes per lane, the rest (128 or 256 bytes)
// with 4 bytes per lane; with 128 bytes, lanes 32..63 repeat lanes 0..31 into the
// 128 bytes after the tile, so nothing outside the tile is fetched.
template <int BYTES>
struct StageShape {
    static constexpr int KB = BYTES / 1024, REST = BYTES % 1024;
    static_assert(REST == 128 || REST == 256, "tile tails of 128 or 256 bytes");
    static constexpr int SIZE = KB * 1024 + 256;  // LDS bytes per stage
};

template <int BYTES>
__device__ __forceinline__ void stage_tile(__amdgpu_buffer_rsrc_t r, uint8_t* stage, int tile_off, int lane) {
    using S = StageShape<BYTES>;
    using lds_ptr = __attribute__((address_space(3))) void*;
#pragma unroll
    for (int k = 0; k < S::KB; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(stage + 1024 * k), 16, 16 * lane, tile_off + 1024 * k, 0,
                                                 kStreamPolicy);
    const int tl = S::REST == 256 ? lane : (lane & 31);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(stage + 1024 * S::KB), 4, 4 * tl, tile_off + 1024 * S::KB, 0,
                                             kStreamPolicy);
}

// ---------------------------------------------------------------------------
// PQ4 keys and values, G = 4 or 8 query heads per KV head, on the bf16 matrix
// cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  Every fp32 operand x
// enters as the pair hi = bf16(x), lo = bf16(x - hi), so the operands carry
// 16 significant bits and the products and sums are exact-in-fp32 MFMA
// arithmetic:
//   scores  D[(h,r)][t] = sum_{j,s} q_r[h][j] * c_s[code_tj]
//           with rows (head h, r = hi/lo of the query), columns 16 tokens and
//           k = (coordinate j, s = hi/lo of the centroid); the score of head h
//           is D[(h,hi)] + D[(h,lo)] times the key block norm;
//   values  D[(h,r)][n] += sum_{t,s} w_r[h][t] * c_s[vcode_t,8n+cb]
//           with columns the 16 code words n of a 128-coordinate block, one
//           accumulator per nibble position cb, k = (token, s).
// Keys go straight from HBM into registers (lane (n, g): code words 4g..4g+3 of
// token n), two register sets alternating between tiles; values go HBM -> LDS
// into two stages per wavefront (distinct LDS objects, so the compiler's wait
// for one stage ignores the other).  The next tile's keys and values are
// requested at the start of the current tile.  Centroid pairs come from 32-entry LDS
// tables (lookup = one SDWA mask and one ds_read_b32), the query pairs from
// LDS (written once per split), and the softmax writes the weight pairs to
// LDS in the A-operand layout of the value products.
template <int D, int G, int TT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(D == 128 ? 4 : 2, D == 128 ? 4 : 2))) void decode_partial_bf16_kernel(DecodeArgs a, DevCodebook cbk, DevCodebook cbv) {
    static_assert(G == 4 || G == 8, "two heads per 16-lane row group");
    using C = Bf16Cfg<D, G, TT>;
    using SM = SmemBf16<D, G, TT>;
    constexpr int VB = C::VB, NB = C::NB, NTB = C::NTB, ROWS = C::ROWS;
    constexpr int STAGE = StageShape<TT * VB>::SIZE;
    __shared__ __align__(16) SM sm;
    __shared__ __align__(16) uint8_t vst0[kWaves][STAGE];
    __shared__ __align__(16) uint8_t vst1[kWaves][STAGE];

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: tile offsets stay in SGPRs
    const int n = lane & 15, g = lane >> 4;  // MFMA column / row (A side) and k-group
    const int hq0 = h * G;
    const int start = s * a.split_len;
    const size_t rec0 = (static_cast<size_t>(b) * a.hq + hq0) * a.splits + s;

    const size_t stream_row = (static_cast<size_t>(b) * a.hkv + h) * a.capacity;
    const uint32_t stream_bytes = static_cast<uint32_t>(a.capacity) * VB;
    const __amdgpu_buffer_rsrc_t krs = stream_rsrc(a.k_cache + stream_row * VB, stream_bytes);
    const __amdgpu_buffer_rsrc_t vrs = stream_rsrc(a.v_cache + stream_row * VB, stream_bytes);
    const __amdgpu_buffer_rsrc_t krs_none = null_rsrc(a.k_cache), vrs_none = null_rsrc(a.v_cache);
    const int k_norm = n * VB;                   // key norm of token n
    const int k_word = n * VB + 4 + 16 * g;      // key words 4g..4g+3 of token n
    uint32_t* wa = sm.u.op.wa[w];

    // the first tile of this wavefront in flight before anything else, before the sequence
    // length arrives (tiles lie inside the cache: t0 + TT <= capacity because TT divides 64; a
    // tile at or past the end is read and not used), its values first: the wait for its keys
    // covers them
    int t0 = start + w * TT;
    KeyTile<NTB, NB> kt[2];
    ValueTile<NTB, NB> vt;
    stage_tile<TT * VB>(vrs, vst0[w], t0 * VB, lane);
    load_keys<VB>(kt[0], krs, k_norm, k_word, t0 * VB);

    if (tid < 32) {
        sm.klo[tid] = bf16_split(cbk.centroids[tid & 15]);
        sm.khi[tid] = bf16_split(cbk.centroids[tid >> 1]);
        sm.vlo[tid] = bf16_split(cbv.centroids[tid & 15]);
        sm.vhi[tid] = bf16_split(cbv.centroids[tid >> 1]);
    }
    if (ROWS < 16 && lane < 16) wa[C::WA - 16 + lane] = 0u;

    // query A operand: row m = n = (head m/2, r = m&1), k-group g holds
    // coordinates 128 blk + 32 g + 4 cc + u (u = 0..3) of chunk c = 8 blk + cc,
    // each as the bf16 half r of q * log2(e)/sqrt(d), duplicated for s = hi/lo.
    {
        const float qscale = kLog2e / sqrtf(static_cast<float>(D));
        const int hm = n >> 1, r = n & 1;
        const float* qg = a.q_rot + (static_cast<size_t>(b) * a.hq + hq0 + (hm < G ? hm : 0)) * D;
#pragma unroll
        for (int c = w; c < NB * 8; c += kWaves) {  // chunks split over the wavefronts
            u32x4 v;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = 128 * (c >> 3) + 32 * g + 4 * (c & 7) + u;
                const uint32_t pr = bf16_split(qg[j] * qscale);
                const uint32_t half = r ? (pr >> 16) : (pr & 0xFFFFu);
                v[u] = n < ROWS ? (half | (half << 16)) : 0u;
            }
            sm.u.op.qa[c][lane] = v;
        }
    }

    int N = a.seq_lens[b];
    N = N < 0 ? 0 : (N > a.capacity ? a.capacity : N);
    const int end = min(start + a.split_len, N);
    if (start >= end) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the staged tile lands before the LDS is released
        for (int gg = 0; gg < G; ++gg) {
            const size_t rec = rec0 + static_cast<size_t>(gg) * a.splits;
            if (tid == 0) a.ml[rec] = make_float2(-INFINITY, 0.0f);
            for (int j = tid; j < D; j += blockDim.x) a.acc[rec * D + j] = 0.0f;
        }
        return;
    }
    lds_write_barrier();  // tables and query operands; the first tile stays in flight

    // d 256 (two waves per SIMD, 256 registers each): the query operand in registers for the
    // whole split (64 of them), not re-read from LDS per tile; d 128 (four waves per SIMD) reads
    // each chunk from LDS a few products ahead of its use
    constexpr bool QREG = D == 256;
    u32x4 qall[QREG ? NB * 8 : 1];
    if constexpr (QREG) {
#pragma unroll
        for (int S = 0; S < NB * 8; ++S) qall[S] = sm.u.op.qa[S][lane];
    }
    // per lane: heads 2g and 2g+1 (when < G); inactive rows keep m = 0, p = 0
    float m_run[2], l_run[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        m_run[e] = (2 * g + e < G) ? -INFINITY : 0.0f;
        l_run[e] = 0.0f;
    }
    f32x4 acc[NB][8];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) acc[blk][cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const char* klo = reinterpret_cast<const char*>(sm.klo);
    const char* khi = reinterpret_cast<const char*>(sm.khi);
    const char* vlo = reinterpret_cast<const char*>(sm.vlo);
    const char* vhi = reinterpret_cast<const char*>(sm.vhi);
    // value-product A operand of this lane: row n (zero row when n >= ROWS), tokens 4g..4g+3
    // with sparse V the reference follows the maximum exactly, so weights against it are as
    // small as they can be and more values drop
    const float slack = a.v_skip > 0.0f ? 0.0f : kRescaleSlack;
    const uint32_t rd_lane = n < ROWS ? n * 16 + 4 * g : C::WA - 16 + 4 * g;
    const uint32_t wa_step = n < ROWS ? ROWS * 16 : 0;  // words per 16-token block
    const uint32_t w_lane = 4 * g * 16 + n;              // this lane's weight word in block 0
    // this lane's value norm and words in a stage (token n; tokens 4g.., word n)
    const uint32_t v_norm_lane = lds_offset(n * VB), v_word_lane = lds_offset(4 * g * VB + 4 + 4 * n);
    constexpr int kStep = kWaves * TT;

    // One tile at t0; P = tile parity selects the key register set and the value stage.
    auto tile = [&](auto pc, const int t0) {
        constexpr int P = decltype(pc)::value;
        KeyTile<NTB, NB>& kc = kt[P];
        const int nv = min(TT, end - t0);  // <= 0 for the odd tile after the last one
        // past the last tile the requests go through the empty resource
        const bool more = t0 + kStep < end;
        const int t_next = more ? t0 + kStep : t0;
        const __amdgpu_buffer_rsrc_t krn = more ? krs : krs_none, vrn = more ? vrs : vrs_none;
        const uint8_t* vcur = P == 0 ? vst0[w] : vst1[w];
        stage_tile<TT * VB>(vrn, P == 0 ? vst1[w] : vst0[w], t_next * VB, lane);
        load_keys<VB>(kt[1 - P], krn, k_norm, k_word, t_next * VB);

        // ---- scores: column n = token 16 tb + n, k-group g = 32 coordinates per
        // block.  Job J = S * NTB + tb multiplies chunk S (nibbles 4(S&1)..+3 of
        // key word (S%8)/2 of block S/8) for token block tb; the lookups run
        // kLookahead jobs ahead of the products, which keeps the LDS results in
        // flight within lgkmcnt's range of 15.
        f32x4 dsc[NTB][NB];
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) dsc[tb][blk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        float nk[NTB][NB];
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) nk[tb][blk] = half_bits_to_float(kc.norm[tb][blk]);
        {
            // (d 128) QB query chunks in flight: chunk S is loaded at job S*NTB and last read by
            // the product of job S*NTB + NTB-1, kLookahead jobs later
            constexpr int NS = NB * 8, NJ = NS * NTB, R = kLookahead + 1, QB = 1 + (kLookahead + NTB - 1) / NTB;
            uint32_t ring[R][4];
            u32x4 qk[QREG ? 1 : QB];
            static_for<NJ + kLookahead>([&](auto jc) {
                constexpr int J = decltype(jc)::value;
                if constexpr (J < NJ) {
                    constexpr int S = J / NTB, TB = J % NTB, BLK = S / 8, CC = S % 8;
                    if constexpr (!QREG && TB == 0) qk[S % QB] = sm.u.op.qa[S][lane];
                    const uint32_t x = kc.w[TB][BLK][CC >> 1];
                    decode_half<CC & 1>(x << 2, x >> 1, klo, khi, ring[J % R]);
                }
                if constexpr (J >= kLookahead) {
                    constexpr int M = J - kLookahead, S = M / NTB, TB = M % NTB, BLK = S / 8;
                    dsc[TB][BLK] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, QREG ? qall[QREG ? S : 0] : qk[S % QB]),
                        __builtin_bit_cast(bf16x8, u32x4{ring[M % R][0], ring[M % R][1], ring[M % R][2], ring[M % R][3]}),
                        dsc[TB][BLK], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);  // keep the issue order written here
            });
        }
        // this tile's value words and norms, from its stage
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
                vt.norm[tb][blk] = *reinterpret_cast<const uint16_t*>(vcur + v_norm_lane + 16 * tb * VB + 68 * blk);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    vt.w[tb][blk][u] =
                        *reinterpret_cast<const uint32_t*>(vcur + v_word_lane + (16 * tb + u) * VB + 68 * blk);
            }

        // ---- online softmax; lane (n, g) holds token 16 tb + n of heads 2g, 2g+1
        // (G is even, so both heads of a lane exist exactly when 2g < G)
        const bool live = 2 * g < G;
        float tv[NTB][2];
        float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            const bool ok = live && 16 * tb + n < nv;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                float sc = 0.0f;
#pragma unroll
                for (int blk = 0; blk < NB; ++blk) sc += nk[tb][blk] * (dsc[tb][blk][2 * e] + dsc[tb][blk][2 * e + 1]);
                tv[tb][e] = ok ? sc : -INFINITY;
                mx[e] = fmaxf(mx[e], tv[tb][e]);
            }
        }
        if (a.scores) {
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    if (tv[tb][e] != -INFINITY)
                        a.scores[(static_cast<size_t>(b) * a.hq + hq0 + 2 * g + e) * a.capacity + t0 + 16 * tb + n] =
                            tv[tb][e] * kLn2;
        }
        if (__builtin_amdgcn_ballot_w64(mx[0] > m_run[0] + slack || mx[1] > m_run[1] + slack) != 0) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float mn = fmaxf(m_run[e], row16_max(mx[e]));
                const float alpha = mn == m_run[e] ? 1.0f : __builtin_amdgcn_exp2f(m_run[e] - mn);  // -inf start gives 0
                l_run[e] *= alpha;
#pragma unroll
                for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                    for (int cb = 0; cb < 8; ++cb) {
                        acc[blk][cb][2 * e] *= alpha;
                        acc[blk][cb][2 * e + 1] *= alpha;
                    }
                m_run[e] = mn;
            }
        }
        float pw[NTB][2][NB];
        bool keep = false;
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            const bool tok = 16 * tb + n < nv;
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
                // rows past the sequence end hold whatever the cache held: their
                // weight must be an exact 0, not 0 * (a stale norm that may be NaN)
                const float nvn = tok ? half_bits_to_float(vt.norm[tb][blk]) : 0.0f;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float p = __builtin_amdgcn_exp2f(tv[tb][e] - m_run[e]);  // 0 for invalid tokens and rows
                    if (blk == 0) l_run[e] += p;
                    pw[tb][e][blk] = (p >= a.v_skip ? p : 0.0f) * nvn;
                    keep = keep || pw[tb][e][blk] != 0.0f;
                }
            }
        }
        // the value products of the tile only where some weight is left (uniform)
        if (__builtin_amdgcn_ballot_w64(keep) == 0) return;
        if (live) {
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int blk = 0; blk < NB; ++blk) {
                        const float wt = pw[tb][e][blk];
                        const uint32_t bits = __float_as_uint(wt);
                        const float lo = wt - __uint_as_float(bits & 0xFFFF0000u);
                        uint32_t* dst = wa + lds_offset(w_lane + ((blk * NTB + tb) * ROWS + 2 * e) * 16);
                        dst[0] = dup_hi16(bits);                 // row (h, hi)
                        dst[16] = dup_hi16(__float_as_uint(lo));  // row (h, lo)
                    }
        }
        lds_order();

        // ---- values: column n = code word n (coordinates 8n..8n+7 of a block),
        // k-group g = tokens 16 tb + 4g + u, one accumulator per nibble position
        // cb.  Job J = (tb, blk, cb): nibble cb of the four tokens' words, four
        // lookups, kLookahead jobs ahead of the products.
        {
            u32x4 av[NTB][NB];
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int blk = 0; blk < NB; ++blk)
                    av[tb][blk] = *reinterpret_cast<const u32x4*>(wa + lds_offset(rd_lane + (blk * NTB + tb) * wa_step));
            constexpr int NJ = NTB * NB * 8, R = kLookahead + 1;
            uint32_t ring[R][4];
            static_for<NJ + kLookahead>([&](auto jc) {
                constexpr int J = decltype(jc)::value;
                if constexpr (J < NJ) {
                    constexpr int TB = J / (8 * NB), BLK = (J / 8) % NB, CB = J % 8;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint32_t x = vt.w[TB][BLK][u];
                        ring[J % R][u] = (CB & 1) ? *reinterpret_cast<const uint32_t*>(vhi + nibble_offset<CB / 2>(x >> 1))
                                                  : *reinterpret_cast<const uint32_t*>(vlo + nibble_offset<CB / 2>(x << 2));
                    }
                }
                if constexpr (J >= kLookahead) {
                    constexpr int M = J - kLookahead, TB = M / (8 * NB), BLK = (M / 8) % NB, CB = M % 8;
                    acc[BLK][CB] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, av[TB][BLK]),
                        __builtin_bit_cast(bf16x8, u32x4{ring[M % R][0], ring[M % R][1], ring[M % R][2], ring[M % R][3]}),
                        acc[BLK][CB], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);  // keep the issue order written here
            });
        }
        lds_order();
    };
    // pairs of tiles, so that the parity is static; the second tile of the last pair may be
    // empty (its weights are all zero, and the running maximum is finite by then)
    for (; t0 < end; t0 += 2 * kStep) {
        tile(std::integral_constant<int, 0>{}, t0);
        tile(std::integral_constant<int, 1>{}, t0 + kStep);
    }
    // the last requests (tiles past the end) land before the LDS is released
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // ---- merge the wavefronts of the workgroup and write the split record
#pragma unroll
    for (int e = 0; e < 2; ++e) l_run[e] = row16_sum(l_run[e]);
    __syncthreads();
    float* red = sm.u.red;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int hh = 2 * g + e;
        if (hh < G) {
            float* r = red + (w * G + hh) * (2 + D);
            if (n == 0) { r[0] = m_run[e]; r[1] = l_run[e]; }
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) r[2 + 128 * blk + 8 * n + cb] = acc[blk][cb][2 * e] + acc[blk][cb][2 * e + 1];
        }
    }
    __syncthreads();
    __shared__ float fw[kWaves * G];
    merge_factors<D, G, kWaves>(red, fw, tid, a.ml + rec0, a.splits);
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += blockDim.x) {
        const int gg = idx / D, j = idx % D;
        const size_t rec = rec0 + static_cast<size_t>(gg) * a.splits;
        a.acc[rec * D + j] = merged_coordinate<D, G, kWaves>(red, fw, gg, j);
    }
}

// ---------------------------------------------------------------------------
// PQ4 at d = 256 with one centroid table for keys and values, G = 4 or 8: the products of
// decode_partial_bf16_kernel with the centroid pairs of a whole code byte per lookup.  A
// 64 KB table maps a byte to (T[low nibble], T[high nibble]) as bf16 (hi, lo) pairs, in 32
// copies (one per lane of a 32-lane phase of the 8-byte LDS reads), 256-byte rows, so that a
// lookup address (byte << 8 | copy << 3) is one byte permute of the code word:
//   * a score product takes the four coordinates of two code bytes: two lookups (the
//     nibble tables take four);
//   * a value lookup gives nibble positions 2c and 2c + 1 of a token's code word, the B
//     operands of two products: four lookups per two products (eight with nibble tables).
// Eight wavefronts per workgroup share the table, one split per workgroup; a wavefront walks
// 32-token tiles as the bf16 kernel does, its query operand held in registers.  A token's
// value weights serve both 128-coordinate blocks: each block of a d 256 vector holds the
// full-vector norm ([P1] section 9, head_dim-specific blocks), so the weights are formed once
// from block 0's norm.
// The keys of a d 256 tile with block 0's norm only (each block holds the full-vector norm).
template <int VB, int NTB, int NB>
__device__ __forceinline__ void load_keys_n0(KeyTile<NTB, NB>& k, __amdgpu_buffer_rsrc_t r, int norm_off, int word_off,
                                             int tile_off) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        k.norm[tb][0] = __builtin_amdgcn_raw_buffer_load_b16(r, norm_off + 16 * tb * VB, tile_off, kStreamPolicy);
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
            k.w[tb][blk] = __builtin_bit_cast(u32x4u, __builtin_amdgcn_raw_buffer_load_b128(r, word_off + 16 * tb * VB + 68 * blk,
                                                                                          tile_off, kStreamPolicy));
    }
}

template <int G>
struct D256Cfg {
    static constexpr int D = 256, NB = 2, VB = 136, TT = 32, NTB = 2, NW = 8, ROWS = 2 * G;
    static constexpr int WA = NTB * ROWS * 16 + (ROWS < 16 ? 16 : 0);  // weight words per wavefront (+ zero row)
};

template <int G>
struct SmemD256 {
    using C = D256Cfg<G>;
    union {
        uint2 tab[256 * 32];                // (byte b, copy c) at b * 32 + c
        float red[C::NW * G * C::D];        // per-wavefront value sums after the tile loop
    } u;
    union {
        alignas(16) uint32_t wa[C::NW][C::WA];  // value-product A operand [tb][row][token] (+ zero row)
        alignas(16) u32x4 qa[16][64];           // score A operand per chunk and lane, until held in registers
    } op;
    float2 ml[C::NW][G];  // per-wavefront (m, l) after the tile loop
    float fw[C::NW * G];  // merge factors
};

template <int G>
__global__ __launch_bounds__(D256Cfg<G>::NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_partial_d256_kernel(
    DecodeArgs a, DevCodebook cb) {
    static_assert(G == 4 || G == 8, "two heads per 16-lane row group");
    using C = D256Cfg<G>;
    constexpr int D = C::D, VB = C::VB, NB = C::NB, NTB = C::NTB, TT = C::TT, NW = C::NW, ROWS = C::ROWS;
    constexpr int STAGE = StageShape<TT * VB>::SIZE;
    static_assert(sizeof(SmemD256<G>::u.red) <= sizeof(SmemD256<G>::u.tab), "the merge fits the table area");
    __shared__ __align__(16) SmemD256<G> sm;
    __shared__ __align__(16) uint8_t vst0[NW][STAGE];
    __shared__ __align__(16) uint8_t vst1[NW][STAGE];

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: tile offsets stay in SGPRs
    const int n = lane & 15, g = lane >> 4;  // MFMA column / row (A side) and k-group
    const int hq0 = h * G;
    const int start = s * a.split_len;
    const size_t rec0 = (static_cast<size_t>(b) * a.hq + hq0) * a.splits + s;

    const size_t stream_row = (static_cast<size_t>(b) * a.hkv + h) * a.capacity;
    const uint32_t stream_bytes = static_cast<uint32_t>(a.capacity) * VB;
    const __amdgpu_buffer_rsrc_t krs = stream_rsrc(a.k_cache + stream_row * VB, stream_bytes);
    const __amdgpu_buffer_rsrc_t vrs = stream_rsrc(a.v_cache + stream_row * VB, stream_bytes);
    const __amdgpu_buffer_rsrc_t krs_none = null_rsrc(a.k_cache), vrs_none = null_rsrc(a.v_cache);
    const int k_norm = n * VB;               // key norm of token n
    const int k_word = n * VB + 4 + 16 * g;  // key words 4g..4g+3 of token n

    // the query entries this thread stages, requested first (the memory counter drains in order:
    // a load behind the tile's would wait for it)
    const float qscale = kLog2e / sqrtf(static_cast<float>(D));
    const int hm = n >> 1, r = n & 1;
    const float* qg = a.q_rot + (static_cast<size_t>(b) * a.hq + hq0 + (hm < G ? hm : 0)) * D;
    float4 qv[NB * 8 / NW];
#pragma unroll
    for (int k = 0; k < NB * 8 / NW; ++k) {
        const int c = w + NW * k;
        qv[k] = *reinterpret_cast<const float4*>(qg + 128 * (c >> 3) + 32 * g + 4 * (c & 7));
    }
    // the first tile before anything else, before the sequence length arrives (a tile past the
    // stream's range reads zeros, one at or past the end is read and not used), its values
    // first: the wait for its keys covers them
    // keys KA tiles ahead of the products (G = 8: two, in three register sets; G = 4, whose
    // zero rows cost registers: one), values one tile ahead in two stages
    constexpr int KA = G == 8 ? 2 : 1, NK = KA + 1, UNR = KA == 2 ? 6 : 2;
    constexpr int kStep = NW * TT;
    int t0 = start + w * TT;
    KeyTile<NTB, NB> kt[NK];
    ValueTile<NTB, NB> vt;
    stage_tile<TT * VB>(vrs, vst0[w], t0 * VB, lane);
    static_for<KA>([&](auto kc) {
        constexpr int K = decltype(kc)::value;
        load_keys_n0<VB>(kt[K], krs, k_norm, k_word, (t0 + K * kStep) * VB);
    });
    __builtin_amdgcn_sched_barrier(0);  // the requests stay ahead of the table and query work

    // table: thread t fills entries t + 512 i, i.e. byte t / 32 + 16 i (low nibble t / 32, high
    // nibble i) in copy t % 32; each store instruction covers 4 KB contiguously
    {
        static_assert(NW * 64 == 512, "the table fill assumes 512 threads");
        uint32_t pc[16], plo = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            pc[i] = bf16_split(cb.centroids[i]);
            plo = (tid >> 5) == i ? pc[i] : plo;  // selected, not indexed: no load of the arguments
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.u.tab[tid + 512 * i] = make_uint2(plo, pc[i]);
    }
    // query A operand: row m = n = (head m/2, r = m&1), k-group g holds coordinates
    // 128 blk + 32 g + 4 cc + u (u = 0..3) of chunk c = 8 blk + cc, each as the bf16 half r of
    // q * log2(e)/sqrt(d), duplicated for the centroid's two halves
    {
#pragma unroll
        for (int k = 0; k < NB * 8 / NW; ++k) {  // chunks split over the wavefronts
            const float qe[4] = {qv[k].x, qv[k].y, qv[k].z, qv[k].w};
            u32x4 v;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t pr = bf16_split(qe[u] * qscale);
                const uint32_t half = r ? (pr >> 16) : (pr & 0xFFFFu);
                v[u] = n < ROWS ? (half | (half << 16)) : 0u;
            }
            sm.op.qa[w + NW * k][lane] = v;
        }
    }

    int N = a.seq_lens[b];
    N = N < 0 ? 0 : (N > a.capacity ? a.capacity : N);
    const int end = min(start + a.split_len, N);
    if (start >= end) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the staged tile lands before the LDS is released
        for (int gg = 0; gg < G; ++gg) {
            const size_t rec = rec0 + static_cast<size_t>(gg) * a.splits;
            if (tid == 0) a.ml[rec] = make_float2(-INFINITY, 0.0f);
            for (int j = tid; j < D; j += blockDim.x) a.acc[rec * D + j] = 0.0f;
        }
        return;
    }
    lds_write_barrier();  // table and query operand; the first tile stays in flight
    u32x4 qall[NB * 8];
#pragma unroll
    for (int S = 0; S < NB * 8; ++S) qall[S] = sm.op.qa[S][lane];
    lds_write_barrier();  // every wavefront holds its query operand before any writes weights there
    uint32_t* wa = sm.op.wa[w];
    if (ROWS < 16 && lane < 16) wa[C::WA - 16 + lane] = 0u;

    // per lane: heads 2g and 2g+1 (when < G); inactive rows keep m = 0, p = 0
    float m_run[2], l_run[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        m_run[e] = (2 * g + e < G) ? -INFINITY : 0.0f;
        l_run[e] = 0.0f;
    }
    f32x4 acc[NB][8];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int cb8 = 0; cb8 < 8; ++cb8) acc[blk][cb8] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const char* tab = reinterpret_cast<const char*>(sm.u.tab);
    const uint32_t lc = (lane & 31) * 8u;  // byte 0 of a lookup address: this lane's copy
    // with sparse V the reference follows the maximum exactly, so weights against it are as
    // small as they can be and more values drop
    const float slack = a.v_skip > 0.0f ? 0.0f : kRescaleSlack;
    // value-product A operand of this lane: row n (zero row when n >= ROWS), tokens 4g..4g+3
    const uint32_t rd_lane = n < ROWS ? n * 16 + 4 * g : C::WA - 16 + 4 * g;
    const uint32_t wa_step = n < ROWS ? ROWS * 16 : 0;  // words per 16-token block
    // this lane's weight word in block 0: token n at the k-group of the 2:4-sparse value product
    // that holds it (token 4 gb + e at group 2 gb + (e & 1) + 8 (e >> 1))
    const uint32_t w_lane = 4 * g * 16 + 2 * (n >> 2) + (n & 1) + 8 * ((n >> 1) & 1);
    // this lane's value norm and words in a stage (token n; tokens 4g.., word n)
    const uint32_t v_norm_lane = lds_offset(n * VB), v_word_lane = lds_offset(4 * g * VB + 4 + 4 * n);

    auto entry = [&](uint32_t word, int byte) __attribute__((always_inline)) {
        return *reinterpret_cast<const uint2*>(tab + __builtin_amdgcn_perm(word, lc, 0x0C0C0400u + (byte << 8)));
    };

    // One tile at t0; I = the tile's index mod UNR: key register set I % NK (the keys of the tile
    // KA ahead go into set (I + KA) % NK), value stage I % 2 (the next tile's values into the other)
    auto tile = [&](auto ic, const int t0) {
        constexpr int I = decltype(ic)::value, P = I % 2, K = I % NK, KN = (I + KA) % NK;
        KeyTile<NTB, NB>& kc = kt[K];
        const int nv = min(TT, end - t0);
        const bool more = t0 + kStep < end, morek = t0 + KA * kStep < end;
        const int t_next = more ? t0 + kStep : t0, t_nextk = morek ? t0 + KA * kStep : t0;
        const uint8_t* vcur = P == 0 ? vst0[w] : vst1[w];
        stage_tile<TT * VB>(more ? vrs : vrs_none, P == 0 ? vst1[w] : vst0[w], t_next * VB, lane);
        load_keys_n0<VB>(kt[KN], morek ? krs : krs_none, k_norm, k_word, t_nextk * VB);

        // ---- scores: job J = S * NTB + tb multiplies chunk S (bytes 2 (S&1), 2 (S&1) + 1 of key
        // word (S%8)/2 of block S/8: four coordinates) for token block tb; the lookups run
        // kLookahead jobs ahead of the products
        f32x4 dsc[NTB][NB];
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) dsc[tb][blk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        float nk[NTB];  // block 0's norm: both blocks hold the vector's norm
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) nk[tb] = half_bits_to_float(kc.norm[tb][0]);
        {
            constexpr int NJ = NB * 8 * NTB, LA = 2, R = LA + 1;
            uint2 ring[R][2];
            static_for<NJ + LA>([&](auto jc) {
                constexpr int J = decltype(jc)::value;
                if constexpr (J < NJ) {
                    constexpr int S = J / NTB, TB = J % NTB, BLK = S / 8, CC = S % 8;
                    const uint32_t x = kc.w[TB][BLK][CC >> 1];
                    ring[J % R][0] = entry(x, 2 * (CC & 1));
                    ring[J % R][1] = entry(x, 2 * (CC & 1) + 1);
                }
                if constexpr (J >= LA) {
                    constexpr int M = J - LA, S = M / NTB, TB = M % NTB, BLK = S / 8;
                    const uint2 e0 = ring[M % R][0], e1 = ring[M % R][1];
                    dsc[TB][BLK] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, qall[S]), __builtin_bit_cast(bf16x8, u32x4{e0.x, e0.y, e1.x, e1.y}),
                        dsc[TB][BLK], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);  // keep the issue order written here
            });
        }
        // this tile's value words, and block 0's norms, from its stage
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            vt.norm[tb][0] = *reinterpret_cast<const uint16_t*>(vcur + v_norm_lane + 16 * tb * VB);
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    vt.w[tb][blk][u] =
                        *reinterpret_cast<const uint32_t*>(vcur + v_word_lane + (16 * tb + u) * VB + 68 * blk);
        }

        // ---- online softmax; lane (n, g) holds token 16 tb + n of heads 2g, 2g+1
        const bool live = 2 * g < G;
        float tv[NTB][2];
        float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            const bool ok = live && 16 * tb + n < nv;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                float sc = 0.0f;
#pragma unroll
                for (int blk = 0; blk < NB; ++blk) sc += dsc[tb][blk][2 * e] + dsc[tb][blk][2 * e + 1];
                tv[tb][e] = ok ? nk[tb] * sc : -INFINITY;
                mx[e] = fmaxf(mx[e], tv[tb][e]);
            }
        }
        if (a.scores) {
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    if (tv[tb][e] != -INFINITY)
                        a.scores[(static_cast<size_t>(b) * a.hq + hq0 + 2 * g + e) * a.capacity + t0 + 16 * tb + n] =
                            tv[tb][e] * kLn2;
        }
        if (__builtin_amdgcn_ballot_w64(mx[0] > m_run[0] + slack || mx[1] > m_run[1] + slack) != 0) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float mn = fmaxf(m_run[e], row16_max(mx[e]));
                const float alpha = mn == m_run[e] ? 1.0f : __builtin_amdgcn_exp2f(m_run[e] - mn);  // -inf start gives 0
                l_run[e] *= alpha;
#pragma unroll
                for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                    for (int cb8 = 0; cb8 < 8; ++cb8) {
                        acc[blk][cb8][2 * e] *= alpha;
                        acc[blk][cb8][2 * e + 1] *= alpha;
                    }
                m_run[e] = mn;
            }
        }
        float pw[NTB][2];
        bool keep = false;
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            // rows past the sequence end hold whatever the cache held: their weight must be an
            // exact 0, not 0 * (a stale norm that may be NaN)
            const float nvn = 16 * tb + n < nv ? half_bits_to_float(vt.norm[tb][0]) : 0.0f;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float p = __builtin_amdgcn_exp2f(tv[tb][e] - m_run[e]);  // 0 for invalid tokens and rows
                l_run[e] += p;
                pw[tb][e] = (p >= a.v_skip ? p : 0.0f) * nvn;
                keep = keep || pw[tb][e] != 0.0f;
            }
        }
        // the value products of the tile only where some weight is left (uniform)
        if (__builtin_amdgcn_ballot_w64(keep) == 0) return;
        if (live) {
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float wt = pw[tb][e];
                    const uint32_t bits = __float_as_uint(wt);
                    const float lo = wt - __uint_as_float(bits & 0xFFFF0000u);
                    uint32_t* dst = wa + lds_offset(w_lane + (tb * ROWS + 2 * e) * 16);
                    dst[0] = dup_hi16(bits);                 // row (h, hi)
                    dst[16] = dup_hi16(__float_as_uint(lo));  // row (h, lo)
                }
        }
        lds_order();

        // ---- values: column n = code word n (coordinates 8n..8n+7 of a block), one accumulator
        // per nibble position, on v_smfmac_f32_16x16x64_bf16 (2:4-sparse A, dense B).  Job J =
        // (tb, blk, c): byte c of the words of tokens 16 tb + 4g + u (u = 0..3), four lookups whose
        // eight dwords are the B operand as loaded (lane group g: dense k-groups 2g, 2g + 1 and
        // 8 + 2g, 9 + 2g, one token each: (c_hi, c_lo) of nibble 2c, then of nibble 2c + 1).  The
        // A operand is the weights of the k-groups' tokens, nonzero at positions 0, 1 of every
        // group for nibble 2c (index 0x4444) and at 2, 3 for nibble 2c + 1 (0xEEEE): two
        // products per job, no register moves.  The lookups run one job ahead of the products.
        {
            u32x4 av[NTB];
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) av[tb] = *reinterpret_cast<const u32x4*>(wa + lds_offset(rd_lane + tb * wa_step));
            constexpr int NJ = NTB * NB * 4, LA = 1, R = LA + 1;
            u32x8 ring[R];
            static_for<NJ + LA>([&](auto jc) {
                constexpr int J = decltype(jc)::value;
                if constexpr (J < NJ) {
                    constexpr int TB = J / (4 * NB), BLK = (J / 4) % NB, CQ = J % 4;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint2 e = entry(vt.w[TB][BLK][u], CQ);
                        ring[J % R][2 * u] = e.x;
                        ring[J % R][2 * u + 1] = e.y;
                    }
                }
                if constexpr (J >= LA) {
                    constexpr int M = J - LA, TB = M / (4 * NB), BLK = (M / 4) % NB, CQ = M % 4;
                    const bf16x16 bop = __builtin_bit_cast(bf16x16, ring[M % R]);
                    acc[BLK][2 * CQ] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, av[TB]), bop,
                                                                                  acc[BLK][2 * CQ], 0x4444, 0, 0);
                    acc[BLK][2 * CQ + 1] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(
                        __builtin_bit_cast(bf16x8, av[TB]), bop, acc[BLK][2 * CQ + 1], 0xEEEE, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);  // keep the issue order written here
            });
        }
        lds_order();
    };
    // UNR tiles per trip, so that both buffer indexes are static; the trip stops after the last tile
    bool go = t0 < end;  // wave-uniform
    while (go) {
        static_for<UNR>([&](auto ic) {
            if (go) {
                tile(ic, t0);
                t0 += kStep;
                go = t0 < end;
            }
        });
    }
    // the last requests (tiles past the end) land before the LDS is released
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // ---- merge the wavefronts ([P2] trick 3: rescale to the common maximum) into the record
#pragma unroll
    for (int e = 0; e < 2; ++e) l_run[e] = row16_sum(l_run[e]);
    __syncthreads();  // every lookup of the workgroup is done: the table area takes the sums
    float* red = sm.u.red;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int hh = 2 * g + e;
        if (hh < G) {
            float* r = red + (w * G + hh) * D;
            if (n == 0) sm.ml[w][hh] = make_float2(m_run[e], l_run[e]);
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                for (int cb8 = 0; cb8 < 8; ++cb8) r[128 * blk + 8 * n + cb8] = acc[blk][cb8][2 * e] + acc[blk][cb8][2 * e + 1];
        }
    }
    __syncthreads();
    if (tid < G) {
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm.ml[ww][tid].x);
        float L = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float2 r = sm.ml[ww][tid];
            const float f = r.x == -INFINITY ? 0.0f : exp2f(r.x - M);
            sm.fw[ww * G + tid] = f;
            L = fmaf(r.y, f, L);
        }
        a.ml[rec0 + static_cast<size_t>(tid) * a.splits] = make_float2(M, L);
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += blockDim.x) {
        const int gg = idx / D, j = idx % D;
        float A = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) A = fmaf(red[(ww * G + gg) * D + j], sm.fw[ww * G + gg], A);
        a.acc[(rec0 + static_cast<size_t>(gg) * a.splits) * D + j] = A;
    }
}

// ---------------------------------------------------------------------------
// o, marked as changed at this point: an address built from it is formed here instead of
// being hoisted out of a loop into a register of its own.
__device__ __forceinline__ uint32_t refresh(uint32_t o) {
    asm volatile("" : "+v"(o));
    return o;
}

// This lane's index in its wavefront, computed where it is used (a volatile asm, so the
// value is not hoisted and held in a register across a loop).
__device__ __forceinline__ int lane_here() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Byte-pair centroid table of the PQ4 sparse-matrix decode.  A lookup decodes
// a whole code byte: entry b of a 256-entry table holds the bf16 (hi, lo)
// pairs of both nibbles, (P[b & 15], P[b >> 4]), 8 bytes read by one
// ds_read_b64.  The table is replicated 32 times so that lane l always reads
// copy l % 32, which sits in its own pair of LDS banks: any byte values, no
// bank conflicts.  Addresses are byte * 256 + 8 * (l % 32); one
// v_mov_b32_sdwa drops the code byte into bits 8..15 of a register whose low
// byte holds the lane part.  One workgroup of 16 wavefronts runs four
// consecutive splits of one KV stream (four wavefronts per split) and shares
// the table and the query operand.
constexpr int kPairSub = 4;                    // splits per workgroup
constexpr int kPairWaves = kPairSub * kWaves;  // wavefronts per workgroup
constexpr int kPairCopies = 32;                // table copies, one per LDS bank pair

// Write byte Q of w into bits 8..15 of addr, keeping its other bits.
#define TQ_PUT_BYTE1(Q)                                                                                   \
    template <>                                                                                           \
    __device__ __forceinline__ void put_byte1<Q>(uint32_t & addr, uint32_t w) {                           \
        asm("v_mov_b32_sdwa %0, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_" #Q           \
            : "+v"(addr) : "v"(w));                                                                       \
    }
template <int Q>
__device__ __forceinline__ void put_byte1(uint32_t& addr, uint32_t w);
TQ_PUT_BYTE1(0)
TQ_PUT_BYTE1(1)
TQ_PUT_BYTE1(2)
TQ_PUT_BYTE1(3)
#undef TQ_PUT_BYTE1

// ---------------------------------------------------------------------------
// PQ4 decode on the 2:4-sparse matrix cores (d = 128, G = 4 or 8; at G = 4
// the values may bring centroids of their own, in a second pair table).
// v_smfmac_f32_16x16x64_bf16 multiplies a
// 16 x 64 A operand with at most two nonzeros in every aligned group of four
// k (stored compressed, their positions in an index register) by a dense
// 64 x 16 B operand, at the issue cost of a dense 16 x 16 x 32 product.
//
// Both contractions take that shape with rows (head h, half r of the hi/lo
// split, coordinate parity p), 16 rows per four heads:
//   * a lookup of code byte m in the byte-pair table yields the k-group
//     (c_hi[2m], c_lo[2m], c_hi[2m+1], c_lo[2m+1]);
//   * row (h, r, p) holds its operand at positions 2p and 2p+1 of every
//     group, so it accumulates coordinate 2m + p with both centroid halves.
// Scores: D[(h,r,p)][t] = sum_m q_r[h][2m+p] c[2m+p, t], 16 coordinate pairs
// per product; head h's score is the sum of its four rows times the key norm.
// Values: D[(h,r,p)][n] = sum_t w_r[h][t] c[2m+p, t], 16 tokens per product,
// column n standing for coordinate pair m = 4n + Q of product Q.  After the
// score products lane (n, g) holds head g's score of token n, and after the
// value products head g's coordinates 8n + 2Q + p, so the online softmax and
// its rescaling never leave the lane.
//
// Operand lane layouts of the instruction (checked on the hardware): A lane
// (row i, group g) holds k = 16g .. 16g+15, value 2q+s being the s-th nonzero
// of group q at the position in index bits 4q+2s .. 4q+2s+1; B lane
// (column n, group g) holds k = 8g .. 8g+7 in elements 0..7 and
// k = 32+8g .. 32+8g+7 in elements 8..15.  Dense k-group gd (four k) thus
// sits in A lane group gd / 4 and in B lane group (gd & 7) / 2, element
// quad (gd & 1) + 2 (gd / 8).
__host__ __device__ constexpr int sp_lane_group(int gd) { return (gd & 7) >> 1; }
__host__ __device__ constexpr int sp_quad(int gd) { return (gd & 1) + 2 * (gd >> 3); }
__host__ __device__ constexpr int sp_group(int gb, int e) { return 2 * gb + (e & 1) + 8 * (e >> 1); }

// lookup jobs (four lookups each) in flight ahead of the product consuming the oldest
constexpr int kSpLookahead = 1;

template <int G>
struct SpCfg {
    static constexpr int D = 128, VB = 68, TT = 32, NTB = TT / 16;
    static constexpr int RB = G / 4;                   // 16-row blocks of (head, r, p)
    // token blocks whose weights are in LDS at once: at G = 8 one (the LDS holds the value
    // stages next to the table only so)
    static constexpr int WTB = G == 8 ? 1 : NTB;
    static constexpr int WA = WTB * G * 2 * 16;         // weight words per wavefront: [tb][head][r][k-group]
    static constexpr int RED = kPairWaves * G * (2 + D);
};

template <int G, bool VTAB, int KF, int VF>
struct SmemSp {
    using C = SpCfg<G>;
    static constexpr bool K3 = KF == TQ_FMT_PQ3, V3 = VF == TQ_FMT_PQ3;
    // PQ3 table bytes are 6-bit indexes (64 entries), PQ4 bytes two 4-bit codes (256)
    static constexpr int KENT = (K3 ? 64 : 256) * kPairCopies;
    static constexpr int VENT = VTAB ? (V3 ? 64 : 256) * kPairCopies : 1;
    static constexpr int NQW = V3 ? 4 : 1;  // value A operands per token block (PQ3: one per block of 32)
    union {
        struct {
            uint2 table[KENT];                       // entry (byte b, copy c) at b * 32 + c
            uint2 vtable[VENT];                      // the values' own table when their centroids differ
            alignas(16) u32x4 qa[C::RB][4][64];      // compressed score A operand per row block, product, lane
            // PQ3 values: per wavefront [tb][token][pair slot j] index words (byte Q: pair j of block Q),
            // token rows of 20 words so the four token quads of a read fall on distinct banks
            alignas(16) uint32_t vidx[V3 ? kPairWaves : 1][V3 ? C::NTB * 16 * 20 : 4];
        } op;
        float red[C::RED];                           // per-wavefront (m, l, acc) after the tile loop
    } u;
    alignas(16) uint32_t wa[kPairWaves][C::WA * NQW];
};

// A value tile of BYTES bytes (a multiple of 256), HBM -> LDS by buffer loads with an
// LDS destination: whole kilobytes with 16 bytes per lane, then 256-byte pieces with 4.
template <int BYTES>
__device__ __forceinline__ void stage_bytes(__amdgpu_buffer_rsrc_t r, uint8_t* stage, int tile_off, int lane) {
    static_assert(BYTES % 256 == 0, "whole 256-byte pieces");
    using lds_ptr = __attribute__((address_space(3))) void*;
    constexpr int KB = BYTES / 1024, R = (BYTES % 1024) / 256;
#pragma unroll
    for (int k = 0; k < KB; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(stage + 1024 * k), 16, 16 * lane, tile_off + 1024 * k, 0,
                                                 kStreamPolicy);
#pragma unroll
    for (int k = 0; k < R; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(stage + 1024 * KB + 256 * k), 4, 4 * lane,
                                                 tile_off + 1024 * KB + 256 * k, 0, kStreamPolicy);
}

// A value tile of whole kilobytes and 128 bytes into exactly that much LDS, 16 bytes per
// lane: the kilobytes with all lanes, the last 128 bytes with lanes 0..7 (one offset
// register serves every load).
template <int BYTES>
__device__ __forceinline__ void stage_tight(__amdgpu_buffer_rsrc_t r, uint8_t* stage, int tile_off, int lane) {
    static_assert(BYTES % 1024 == 128, "whole kilobytes and 128 bytes");
    using lds_ptr = __attribute__((address_space(3))) void*;
    constexpr int KB = BYTES / 1024;
#pragma unroll
    for (int k = 0; k < KB; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(stage + 1024 * k), 16, 16 * lane, tile_off + 1024 * k, 0,
                                                 kStreamPolicy);
    if (lane < 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(stage + 1024 * KB), 16, 16 * lane, tile_off + 1024 * KB, 0,
                                                 kStreamPolicy);
}

// ---------------------------------------------------------------------------
// turbo3 (PQ3) blocks on the same matrix products.  A 32-coordinate PQ3 block ([fp16 norm]
// [8 bytes of low bit pairs][4 bytes of high bits], [P1] sections 2 and 4) is the slice of a
// vector that one lane group of a score product covers, so a lane loads one block of one
// token (16 bytes at the block's 4-byte-aligned start) and turns each run of 8 coordinates
// into a word of four table indexes, one per coordinate pair: the pair's two low bit pairs
// in bits 0-3 and its two high bits in bits 4-5 (a 64-entry table gives both centroids).
// Each block has its own norm, so every product must cover one block: a transpose across
// the four lane groups (two lane-swap steps) gives lane group g run g of every block.

// Index word of a run: lo = its low bits placed by a byte permute as [b0, 0, b1, 0]
// (coordinate e of the run at bits 2e of b1:b0), hi = its high-bit byte (coordinate e at
// bit e) alone in bits 0-7.
__device__ __forceinline__ uint32_t pq3_index_word(uint32_t lo, uint32_t hi) {
    lo = ((lo << 4) | lo) & 0x0F0F0F0Fu;    // nibble k (pair k's low bits) in byte k
    hi = ((hi << 12) | hi) & 0x000F000Fu;   // pairs 0, 1 in bits 0-3, pairs 2, 3 in bits 16-19
    hi = ((hi << 6) | hi) & 0x03030303u;    // pair k's high bits in bits 0-1 of byte k
    return (hi << 4) | lo;
}

// Byte-permute selectors of a lane whose block starts off = 0 or 2 bytes into its aligned
// 16 bytes r0..r3: run s's two low-bit bytes (block bytes 2 + 2s, 3 + 2s) out of (r1:r0)
// for s = 0, 1 and (r2:r1) for s = 2, 3, and its high-bit byte (block byte 10 + s) out of (r3:r2).
struct Pq3Sel {
    uint32_t lo_a, lo_b, hi0;
};
__device__ __forceinline__ Pq3Sel pq3_selectors(uint32_t off) {
    const uint32_t a = off + 2, b = off + 4;
    return {0x0C000C00u | a | (a + 1) << 16, 0x0C000C00u | b | (b + 1) << 16, 0x0C0C0C00u | (off + 2)};
}

// The four index words (runs 0..3) and the fp16 norm bits of the block in r.
__device__ __forceinline__ void pq3_block(const u32x4u& r, const Pq3Sel& sel, uint32_t off8, uint32_t (&w)[4],
                                          uint32_t& norm) {
    norm = __builtin_amdgcn_ubfe(r[0], off8, 16);
    w[0] = pq3_index_word(__builtin_amdgcn_perm(r[1], r[0], sel.lo_a), __builtin_amdgcn_perm(r[3], r[2], sel.hi0));
    w[1] = pq3_index_word(__builtin_amdgcn_perm(r[1], r[0], sel.lo_b),
                          __builtin_amdgcn_perm(r[3], r[2], sel.hi0 + 1));
    w[2] = pq3_index_word(__builtin_amdgcn_perm(r[2], r[1], sel.lo_a),
                          __builtin_amdgcn_perm(r[3], r[2], sel.hi0 + 2));
    w[3] = pq3_index_word(__builtin_amdgcn_perm(r[2], r[1], sel.lo_b),
                          __builtin_amdgcn_perm(r[3], r[2], sel.hi0 + 3));
}

// 4 x 4 transpose across the lane groups (rows of 16 lanes): on return x[i] of lane group
// g holds what x[g] of lane group i held.
__device__ __forceinline__ void group_transpose(uint32_t (&x)[4]) {
    const auto a = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    x[0] = c[0];
    x[1] = c[1];
    x[2] = d[0];
    x[3] = d[1];
}

// x of lane group i, for i = 0..3, in every lane group
__device__ __forceinline__ void group_broadcast(uint32_t x, uint32_t (&out)[4]) {
    const auto a = __builtin_amdgcn_permlane32_swap(x, x, false, false);  // [x0 x1 x0 x1], [x2 x3 x2 x3]
    const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[0], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[1], a[1], false, false);
    out[0] = b[0];
    out[1] = b[1];
    out[2] = c[0];
    out[3] = c[1];
}

// 4 x 4 byte transpose inside a lane: byte q of out[k] is byte k of x[q].
__device__ __forceinline__ void byte_transpose(const uint32_t (&x)[4], uint32_t (&out)[4]) {
    const uint32_t p01 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);  // x0b0 x1b0 x0b1 x1b1
    const uint32_t p23 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
    const uint32_t q01 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);  // x0b2 x1b2 x0b3 x1b3
    const uint32_t q23 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
    out[0] = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
    out[1] = __builtin_amdgcn_perm(p23, p01, 0x07060302u);
    out[2] = __builtin_amdgcn_perm(q23, q01, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(q23, q01, 0x07060302u);
}

template <int G, bool VTAB, int KF = TQ_FMT_PQ4, int VF = TQ_FMT_PQ4>
__global__ __launch_bounds__(kPairWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void decode_partial_sparse_kernel(
    DecodeArgs a, DevCodebook cbk, DevCodebook cbv) {
    static_assert(G == 4 || G == 8, "four heads per 16-row block");
    static_assert(!VTAB || G == 4, "two tables fit the LDS at G = 4 only");
    using C = SpCfg<G>;
    constexpr int D = C::D, NTB = C::NTB, RB = C::RB, TT = C::TT;
    constexpr bool K3 = KF == TQ_FMT_PQ3, V3 = VF == TQ_FMT_PQ3, PQ4PAIR = !K3 && !V3;
    constexpr int VBK = K3 ? 56 : 68, VBV = V3 ? 56 : 68;  // bytes per token of keys and values
    // values through LDS where the two stages fit next to the table (one table; at G = 8 with
    // stages of exactly a tile and the weights of one token block at a time); PQ3 values
    // instead come through registers (two tile buffers) and an LDS index tile
    constexpr bool VLDS = !VTAB;
    static_assert(!V3 || (VLDS && K3), "PQ3 values with PQ3 keys and one table");
    static_assert(PQ4PAIR || G == 4, "PQ3 at four query heads per KV head");
    constexpr bool STAGED = VLDS && !V3;  // value stages filled by buffer-to-LDS loads
    constexpr bool TIGHT = G == 8;        // stages of exactly TT * VBV bytes
    constexpr int STAGE = TIGHT ? TT * VBV : StageShape<TT * (V3 ? 68 : VBV)>::SIZE;  // (no stages with PQ3 values)
    constexpr int WTB = C::WTB;
    // G = 8: score products token block by token block (see the tile's scores), and a few lane
    // offsets formed in the tile instead of held across the tile loop
    constexpr bool TBMAJ = RB == 2;
    __shared__ __align__(16) SmemSp<G, VTAB, KF, VF> sm;
    // two stages in distinct LDS objects: the compiler's wait for one stage's loads then
    // ignores the other stage's
    __shared__ __align__(16) uint8_t vst0[STAGED ? kPairWaves : 1][STAGED ? STAGE : 16];
    __shared__ __align__(16) uint8_t vst1[STAGED ? kPairWaves : 1][STAGED ? STAGE : 16];
    // the rotated query heads of the group, when the kernel rotates the query itself (G = 4)
    __shared__ __align__(16) float qrot_sh[G == 4 ? G : 1][G == 4 ? D : 4];
    // key and value boundaries of the encoder, when the kernel appends the step's token
    __shared__ __align__(16) float app_sb[2][4][4];
    __shared__ uint32_t tail_flag;  // this workgroup finished its stream last

    const int h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wi = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: tile offsets stay in SGPRs
    const int sg = wi / kWaves, w = wi % kWaves;     // split within the workgroup, wavefront within the split
    const int s = blockIdx.x * kPairSub + sg;
    const int n = lane & 15, g = lane >> 4;
    const int hq0 = h * G;
    int N = a.seq_lens[b];
    N = N < 0 ? 0 : (N > a.capacity ? a.capacity : N);
    const int start = s * a.split_len;
    const int end = s < a.splits ? min(start + a.split_len, N) : start;  // no tokens past the last split

    const size_t stream_row = (static_cast<size_t>(b) * a.hkv + h) * a.capacity;
    const __amdgpu_buffer_rsrc_t krs =
        stream_rsrc(a.k_cache + stream_row * VBK, static_cast<uint32_t>(a.capacity) * VBK);
    const __amdgpu_buffer_rsrc_t vrs =
        stream_rsrc(a.v_cache + stream_row * VBV, static_cast<uint32_t>(a.capacity) * VBV);
    const __amdgpu_buffer_rsrc_t krs_none = null_rsrc(a.k_cache), vrs_none = null_rsrc(a.v_cache);
    // PQ4 keys: the norm and code words 4g..4g+3 of token n.  PQ3 keys and values: block g
    // of token n, from the 4-byte-aligned start of its 14 bytes (p3_off bytes before it; a
    // token's 56 bytes start aligned, so blocks 1 and 3 start 2 bytes into a dword)
    const uint32_t p3_off = (14u * g) & 3u;
    const int p3_word = n * 56 + 14 * g - static_cast<int>(p3_off);
    const int k_norm = n * VBK, k_word = K3 ? p3_word : n * VBK + 4 + 16 * g;
    const int v_norm = n * VBV, v_word = 4 * g * VBV + 4 + 4 * n;
    const Pq3Sel p3_sel = pq3_selectors(p3_off);
    uint32_t* wa = sm.wa[wi];
    // the keys of a tile: PQ4 through load_keys, PQ3 one 16-byte block per token block
    auto p3_load = [&](KeyTile<NTB, 1>& k, __amdgpu_buffer_rsrc_t r, int tile_off) __attribute__((always_inline)) {
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
            k.w[tb][0] = __builtin_bit_cast(u32x4u, __builtin_amdgcn_raw_buffer_load_b128(r, p3_word + 16 * tb * 56,
                                                                                         tile_off, kStreamPolicy));
    };
    auto keys_in = [&](KeyTile<NTB, 1>& k, __amdgpu_buffer_rsrc_t r, int tile_off) __attribute__((always_inline)) {
        if constexpr (K3) p3_load(k, r, tile_off);
        else load_keys<VBK>(k, r, k_norm, k_word, tile_off);
    };

    // The small global reads of the prologue come first: a tile load issued before them would
    // have to complete before their values can be used (the memory counter drains in order).
    //   * table entries: thread t writes entries t + 1024 k (k = 0..7) of every table, so each
    //     store instruction covers 512 contiguous bytes (no bank conflicts); entry i is byte
    //     i / 32, whose low nibble is the same for all k and whose high nibble is t / 512 + 2k;
    //   * compressed score A operand: wavefront wi < 4 RB builds product I = wi % 4 of row block
    //     wi / 4; lane (row n, group g) holds, per group q, the pair (q_r, q_r) of coordinate
    //     2m + p, where m is the code byte that B lane group sp_lane_group(4g + q) reads as
    //     element quad sp_quad(4g + q).
    //     PQ3 tables hold bytes 0..63 (k = 0, 1): byte i / 32 = t / 32 + 32 k has the first
    //     code (t / 32) % 4 + 4 ((t / 512) % 2), the same for both k, and the second
    //     (t / 128) % 4 + 4 k;
    static_assert(kPairWaves * 64 == 1024, "the table fill assumes 1024 threads");
    constexpr int KFILL = K3 ? 2 : 8, VFILL = V3 ? 2 : 8;
    const int tb5 = tid >> 5;
    auto code0 = [&](bool pq3) { return pq3 ? (tb5 & 3) | ((tb5 >> 4) & 1) << 2 : tb5 & 15; };
    auto code1 = [&](bool pq3, int k) { return pq3 ? ((tb5 >> 2) & 3) | k << 2 : (tb5 >> 4) + 2 * k; };
    float ck_lo = cbk.centroids[code0(K3)], ck_hi[KFILL], cv_lo = 0.0f, cv_hi[VFILL];
#pragma unroll
    for (int k = 0; k < KFILL; ++k) ck_hi[k] = cbk.centroids[code1(K3, k)];
    if constexpr (VTAB) {
        cv_lo = cbv.centroids[code0(V3)];
#pragma unroll
        for (int k = 0; k < VFILL; ++k) cv_hi[k] = cbv.centroids[code1(V3, k)];
    }
    // an unrotated query (values through LDS only): wavefronts wi < G / 4 rotate it below,
    // four heads each, with the arithmetic of the query rotation kernel (16 lanes per head,
    // 8 coordinates per lane: signs, Walsh-Hadamard butterflies, 1/sqrt(d)), so the rotated
    // values are the same bits.  The query and its sign word are read here, before the tiles.
    const bool raw = G == 4 && VLDS && PQ4PAIR && a.q_raw != nullptr;  // uniform
    const int rh = 4 * wi + (lane >> 4), rl = lane & 15;
    float rv[8];
    uint32_t rsign = 0;
    if (raw && wi < G / 4) {
        const float4* src =
            reinterpret_cast<const float4*>(a.q_raw + (static_cast<size_t>(b) * a.hq + hq0 + rh) * D + 8 * rl);
        const float4 p0 = src[0], p1 = src[1];
        rv[0] = p0.x; rv[1] = p0.y; rv[2] = p0.z; rv[3] = p0.w;
        rv[4] = p1.x; rv[5] = p1.y; rv[6] = p1.z; rv[7] = p1.w;
        rsign = cbk.sign_bits[rl >> 2] >> (8 * (rl & 3));  // bits of coordinates 8 rl .. 8 rl + 7
    }
    // the step's new token (values through LDS only): the workgroup whose splits hold position
    // new_pos[b] of this stream encodes its key and value rows with the write kernel's
    // arithmetic (wavefront 1: lanes 0..7 the key, 8..15 the value) and writes them into the
    // caches before any wavefront requests the tile holding them: ahead of the first tiles
    // when the position lies in one, else before the barrier that precedes every other tile.
    bool app = false, app_first = false;
    int apos = 0;
    if (G == 4 && VLDS && PQ4PAIR && a.new_pos != nullptr) {
        apos = a.new_pos[b];
        if (apos >= 0 && apos < a.capacity) {
            const int sp = min(apos / a.split_len, a.splits - 1);
            app = sp / kPairSub == static_cast<int>(blockIdx.x);
            app_first = app && apos - sp * a.split_len < kWaves * TT;
        }
    }
    const bool app_lane = app && wi == 1 && lane < 16, app_v = lane >= 8;
    const int al = lane & 7;
    uint4 araw[2];
    if (app_lane) {
        const uint16_t* src = (app_v ? a.v_new : a.k_new) + (static_cast<size_t>(b) * a.hkv + h) * D + 16 * al;
        araw[0] = reinterpret_cast<const uint4*>(src)[0];
        araw[1] = reinterpret_cast<const uint4*>(src)[1];
    }
    auto append_token = [&]() __attribute__((always_inline)) {
        if (wi != 1) return;
        if (lane < 32)  // boundaries b0 .. b14 and +inf of the key (lanes 0..15) and value tables
            app_sb[lane >> 4][(lane & 15) >> 2][lane & 3] =
                (lane & 15) < 15 ? (lane < 16 ? cbk.bounds[lane & 15] : cbv.bounds[lane & 15]) : INFINITY;
        lds_order();
        if (lane < 16) {
            // the 16 signs of coordinates 16 al .. 16 al + 15 by 64-bit shifts (no indexing)
            const uint64_t s01 = (static_cast<uint64_t>(app_v ? cbv.sign_bits[1] : cbk.sign_bits[1]) << 32) |
                                 (app_v ? cbv.sign_bits[0] : cbk.sign_bits[0]);
            const uint64_t s23 = (static_cast<uint64_t>(app_v ? cbv.sign_bits[3] : cbk.sign_bits[3]) << 32) |
                                 (app_v ? cbv.sign_bits[2] : cbk.sign_bits[2]);
            uint32_t smask[8];
            pq4_sign_masks<16>(static_cast<uint32_t>((al < 4 ? s01 : s23) >> (16 * (al & 3))) & 0xFFFFu, smask);
            const float b3 = app_v ? cbv.bounds[3] : cbk.bounds[3], b7 = app_v ? cbv.bounds[7] : cbk.bounds[7],
                        b11 = app_v ? cbv.bounds[11] : cbk.bounds[11];
            uint32_t n16, words[2];
            pq4_encode<128, 8>(araw, smask, b3, b7, b11, reinterpret_cast<const float4*>(app_sb[app_v ? 1 : 0]), al,
                               n16, words);
            uint8_t* out = (app_v ? a.v_wr : a.k_wr) + ((static_cast<size_t>(b) * a.hkv + h) * a.capacity + apos) * 68;
            pq4_store<128, 8>(out, al, n16, words);
        }
    };
    if (app_first) {
        append_token();
        __syncthreads();  // the rows are in memory before any tile request
    }
    float qv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const int qrb = wi / 4, qI = wi % 4, qhh = 4 * qrb + (n >> 2), qr = (n >> 1) & 1, qp = n & 1;
    if (!raw && wi < 4 * RB) {
        const float* qg = a.q_rot + (static_cast<size_t>(b) * a.hq + hq0 + qhh) * D;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int gd = 4 * g + q;
            // the code byte (coordinate pair) that B lane group sp_lane_group(gd) reads as quad
            // sp_quad(gd) of product qI: PQ4 word qI of its code group, PQ3 run g of block qI
            const int m = K3 ? 16 * qI + 4 * sp_lane_group(gd) + sp_quad(gd)
                             : 16 * sp_lane_group(gd) + 4 * qI + sp_quad(gd);
            qv[q] = qg[2 * m + qp];
        }
    }

    // the first tile, requested unconditionally so the loads stay on one path and the waits of
    // the table fill below count only the small reads above; a wavefront without tiles requests
    // it through the empty resource (zeros, no memory read)
    int t0 = start + w * TT;
    KeyTile<NTB, 1> kt[VLDS ? 2 : 1];
    KeyTile<NTB, 1> vraw[V3 ? 2 : 1];  // PQ3 value blocks, loaded as the keys are
    ValueTile<NTB, 1> vt;
    {
        const bool any = t0 < end;
        const __amdgpu_buffer_rsrc_t kr0 = any ? krs : krs_none, vr0 = any ? vrs : vrs_none;
        keys_in(kt[0], kr0, t0 * VBK);
        if constexpr (V3) p3_load(vraw[0], vr0, t0 * VBV);
        else if constexpr (TIGHT) stage_tight<TT * VBV>(vr0, vst0[wi], t0 * VBV, lane);
        else if constexpr (VLDS) stage_tile<TT * VBV>(vr0, vst0[wi], t0 * VBV, lane);
        else load_values<VBV>(vt, vr0, v_norm, v_word, t0 * VBV);
    }
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int k = 0; k < KFILL; ++k) sm.u.op.table[tid + 1024 * k] = make_uint2(bf16_split(ck_lo), bf16_split(ck_hi[k]));
    if constexpr (VTAB) {
#pragma unroll
        for (int k = 0; k < VFILL; ++k)
            sm.u.op.vtable[tid + 1024 * k] = make_uint2(bf16_split(cv_lo), bf16_split(cv_hi[k]));
    }
    if (app && !app_first) append_token();  // its tile is requested after the barrier below
    if (raw) {
        if (wi < G / 4) {
#pragma unroll
            for (int e = 0; e < 8; ++e) rv[e] *= ((rsign >> e) & 1u) ? -1.0f : 1.0f;
            wht8<16>(rv, rl);
#pragma unroll
            for (int e = 0; e < 8; ++e) qrot_sh[rh][8 * rl + e] = rv[e] * 0.08838834764831845f;  // 1/sqrt(128)
        }
        __syncthreads();
        if (wi < 4 * RB) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int gd = 4 * g + q;
                qv[q] = qrot_sh[qhh][2 * (16 * sp_lane_group(gd) + 4 * qI + sp_quad(gd)) + qp];
            }
        }
    }
    if (wi < 4 * RB) {
        const float qscale = kLog2e / sqrtf(static_cast<float>(D));
        u32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t pr = bf16_split(qv[q] * qscale);
            const uint32_t half = qr ? (pr >> 16) : (pr & 0xFFFFu);
            v[q] = half | (half << 16);
        }
        sm.u.op.qa[qrb][qI][lane] = v;
    }
    __syncthreads();

    // row parity p = n & 1: nonzeros at positions 2p, 2p+1 of every group of four
    const int sp_idx = (n & 1) ? 0xEEEE : 0x4444;
    u32x4 qreg[RB == 1 ? 4 : 1];
    if constexpr (RB == 1) {
#pragma unroll
        for (int I = 0; I < 4; ++I) qreg[I] = sm.u.op.qa[0][I][lane];
    }

    float m_run[RB], l_run[RB];
    f32x4 acc[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.0f;
#pragma unroll
        for (int Q = 0; Q < 4; ++Q) acc[rb][Q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    const char* tab = reinterpret_cast<const char*>(sm.u.op.table);
    const char* vtab = VTAB ? reinterpret_cast<const char*>(sm.u.op.vtable) : tab;
    uint32_t addr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) addr[i] = (lane & 31) * 8u;  // bits 8..15 take the code byte
    // weights: token n is written to k-group sp_group(n / 4, n % 4) of [tb][head][r]; the value
    // A operand of lane (row n, group g) is the four groups 4g .. 4g+3 of its (head, r)
    // with sparse V the reference follows the maximum exactly, so weights against it are as
    // small as they can be and more values drop (not in the kernels that hold the values in
    // registers: the register costs them a spill)
    const float slack = VLDS && a.v_skip > 0.0f ? 0.0f : kRescaleSlack;
    // (lane parts of LDS word offsets, kept whole once so per-tile constants fold into the
    // instructions' offset fields)
    const uint32_t w_lane = lds_offset<VLDS>(g * 32 + sp_group(n >> 2, n & 3));
    const uint32_t rd_lane = lds_offset<VLDS>(((n >> 2) * 2 + ((n >> 1) & 1)) * 16 + 4 * g);
    // PQ3 value index tile: lane (n, g) writes words 4g .. 4g+3 of token n's row and reads word n
    // of the rows of tokens 4g .. 4g+3
    const uint32_t vi_wr = lds_offset(n * 20 + 4 * g), vi_rd = lds_offset(4 * g * 20 + n);
    constexpr int kStep = kWaves * TT;
    constexpr int LA = kSpLookahead, R = LA + 1;
    const uint8_t* vcur = nullptr;  // the value stage of the tile in progress
    // lane parts of this lane's value norm and words in a stage (G = 8: marked as changed in
    // every tile, so that each stage's address is formed there and not held per stage)
    const uint32_t vn_lane = lds_offset(n * VBV), vw_lane = lds_offset(4 * g * VBV + 4 + 4 * n);
    uint32_t vw_here = vw_lane;
    // code words n of tokens 16 tb + 4g .. +3 of the tile in progress, from its stage
    auto read_vwords = [&](int tb) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            vt.w[tb][0][u] = TBMAJ ? *reinterpret_cast<const uint32_t*>(vcur + vw_here + (16 * tb + u) * VBV)
                                   : *reinterpret_cast<const uint32_t*>(vcur + (16 * tb + 4 * g + u) * VBV + 4 + 4 * n);
    };

    // One tile of TT tokens at t0.  With values through LDS the tiles alternate between
    // two key register sets and two value stages (P = tile parity): the next tile's keys
    // and values are requested before this tile's scores.  Otherwise the next keys are
    // requested after the scores and the next values after the value products.
    auto tile = [&](auto pc, const int t0) {
        constexpr int P = decltype(pc)::value;
        KeyTile<NTB, 1>& kc = kt[VLDS ? P : 0];
        const int nv = min(TT, end - t0);  // <= 0 for the odd tile after the last one
        const bool more = t0 + kStep < end;
        const int t_next = more ? t0 + kStep : t0;
        const __amdgpu_buffer_rsrc_t krn = more ? krs : krs_none, vrn = more ? vrs : vrs_none;
        vcur = P == 0 ? vst0[wi] : vst1[wi];
        if constexpr (VLDS) {
            if constexpr (V3) p3_load(vraw[1 - P], vrn, t_next * VBV);
            else if constexpr (TIGHT) stage_tight<TT * VBV>(vrn, P == 0 ? vst1[wi] : vst0[wi], t_next * VBV, lane);
            else stage_tile<TT * VBV>(vrn, P == 0 ? vst1[wi] : vst0[wi], t_next * VBV, lane);
            keys_in(kt[1 - P], krn, t_next * VBK);
        }

        // ---- scores: job J = I * NTB + tb reads bytes 0..3 of key word I of block tb
        // PQ4: the four products of a token block accumulate in dsc.  PQ3: one product per
        // block of 32 coordinates, each from zero into a ring slot and folded into sacc with its
        // block's norm after the next job's lookups (so no fold waits on a product in flight).
        // G = 8 (two row blocks, no query operand in registers): job J = tb * 4 + I, and a token
        // block's scores are folded into sacc once the next block's first product is issued,
        // which keeps one block's accumulators live instead of all
        f32x4 dsc[NTB][RB], dring[K3 ? 3 : 1][RB];
        float sacc[NTB][RB];
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                dsc[tb][rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                sacc[tb][rb] = 0.0f;
            }
        // this lane's four code words of each token block (PQ3: the index words of run g of
        // blocks 0..3) and the key norms of its token (PQ3: of blocks 0..3)
        // (PQ3: fp16 norms of blocks 0..3, token blocks 0 and 1 in the low and high halves)
        uint32_t kw[NTB][4], knorm[4];
        float nk[NTB];
        if constexpr (K3) {
            static_assert(NTB == 2, "two token blocks share one norm word");
            uint32_t nb[NTB];
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                pq3_block(kc.w[tb][0], p3_sel, 8u * p3_off, kw[tb], nb[tb]);
                group_transpose(kw[tb]);
            }
            group_broadcast(nb[0] | nb[1] << 16, knorm);
        } else {
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) kw[tb][i] = kc.w[tb][0][i];
                nk[tb] = half_bits_to_float(kc.norm[tb][0]);
            }
        }
        {
            constexpr int NJ = 4 * NTB;
            u32x8 ring[R];
            // fold product M of a PQ3 key tile: its block's norm times its row-summed column
            auto fold = [&](auto mc) __attribute__((always_inline)) {
                constexpr int M = decltype(mc)::value, I = M / NTB, TB = M % NTB;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const f32x4 d4 = dring[M % 3][rb];
                    const float nrm = half_bits_to_float((knorm[I] >> (16 * TB)) & 0xFFFFu);
                    sacc[TB][rb] = fmaf(nrm, (d4[0] + d4[1]) + (d4[2] + d4[3]), sacc[TB][rb]);
                }
            };
            // fold token block TB of a G = 8 tile: its key norm times its row-summed columns
            auto fold_tb = [&](auto tc) __attribute__((always_inline)) {
                constexpr int TB = decltype(tc)::value;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const f32x4 d4 = dsc[TB][rb];
                    sacc[TB][rb] = nk[TB] * ((d4[0] + d4[1]) + (d4[2] + d4[3]));
                }
            };
            static_for<NJ + LA + (K3 ? 1 : 0)>([&](auto jc) {
                constexpr int J = decltype(jc)::value;
                if constexpr (J < NJ) {
                    constexpr int I = TBMAJ ? J % 4 : J / NTB, TB = TBMAJ ? J / 4 : J % NTB;
                    const uint32_t x = kw[TB][I];
                    put_byte1<0>(addr[0], x);
                    put_byte1<1>(addr[1], x);
                    put_byte1<2>(addr[2], x);
                    put_byte1<3>(addr[3], x);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint2 v = *reinterpret_cast<const uint2*>(tab + addr[e]);
                        ring[J % R][2 * e] = v.x;
                        ring[J % R][2 * e + 1] = v.y;
                    }
                }
                if constexpr (K3 && J >= LA + 2) fold(std::integral_constant<int, J - LA - 2>{});
                if constexpr (J >= LA && J < NJ + LA) {
                    constexpr int M = J - LA, I = TBMAJ ? M % 4 : M / NTB, TB = TBMAJ ? M / 4 : M % NTB;
                    // the previous token block's accumulators are folded before this block's
                    // first product, so the two sets never live at once
                    if constexpr (TBMAJ && I == 0 && TB > 0) fold_tb(std::integral_constant<int, TB - 1>{});
                    const bf16x16 bop = __builtin_bit_cast(bf16x16, ring[M % R]);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        const u32x4 aop = RB == 1 ? qreg[RB == 1 ? I : 0] : sm.u.op.qa[rb][I][lane];
                        if constexpr (K3)
                            dring[M % 3][rb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(
                                __builtin_bit_cast(bf16x8, aop), bop, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, sp_idx, 0, 0);
                        else
                            dsc[TB][rb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, aop), bop,
                                                                                   dsc[TB][rb], sp_idx, 0, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (K3) fold(std::integral_constant<int, NJ - 1>{});  // (NJ - 2 folded in the last job)
            if constexpr (TBMAJ) fold_tb(std::integral_constant<int, NTB - 1>{});
        }
        if constexpr (!VLDS) keys_in(kt[0], krn, t_next * VBK);
        // PQ3 value norms of token 16 tb + n, blocks 0..3 (fp16, token blocks in the two halves)
        uint32_t vnorm[4];
        if constexpr (V3) {
            // this tile's value blocks as index words: lane (n, g) turns block g of token n into
            // the words of pairs 4g .. 4g+3 of all four blocks (byte Q: block Q) and stores them
            // in token n's row; lane (n, g) then reads word n of tokens 4g .. 4g+3, whose byte Q
            // the value product for block Q looks up
            uint32_t* vi = sm.u.op.vidx[wi];
            uint32_t nb[NTB];
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                uint32_t x[4], t4[4];
                pq3_block(vraw[P].w[tb][0], p3_sel, 8u * p3_off, x, nb[tb]);
                nb[tb] = 16 * tb + n < nv ? nb[tb] : 0u;  // past the end: norm 0 (the bits may be NaN)
                group_transpose(x);
                byte_transpose(x, t4);
                *reinterpret_cast<u32x4*>(vi + vi_wr + 16 * 20 * tb) = u32x4{t4[0], t4[1], t4[2], t4[3]};
            }
            group_broadcast(nb[0] | nb[1] << 16, vnorm);
            lds_order();
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int u = 0; u < 4; ++u) vt.w[tb][0][u] = vi[vi_rd + (16 * tb + u) * 20];
        } else if constexpr (VLDS) {  // this tile's value norms and words, from its stage
            const uint32_t vn_here = TBMAJ ? refresh(vn_lane) : 0u;
            if constexpr (TBMAJ) vw_here = refresh(vw_lane);
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                vt.norm[tb][0] = TBMAJ ? *reinterpret_cast<const uint16_t*>(vcur + vn_here + 16 * tb * VBV)
                                       : *reinterpret_cast<const uint16_t*>(vcur + (16 * tb + n) * VBV);
                if constexpr (WTB == NTB) read_vwords(tb);  // (else in the value pass of the block)
            }
        }

        // ---- online softmax: lane (n, g) owns head 4 rb + g, token 16 tb + n
        // (at G = 8 n is recomputed here rather than held across the tile loop)
        const int nt = TBMAJ ? (lane_here() & 15) : n;
        float tv[NTB][RB];
        float mx[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) mx[rb] = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            const bool ok = 16 * tb + nt < nv;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const f32x4 d4 = dsc[tb][rb];
                const float sc = K3 || TBMAJ ? sacc[tb][rb] : nk[tb] * ((d4[0] + d4[1]) + (d4[2] + d4[3]));
                tv[tb][rb] = ok ? sc : -INFINITY;
                mx[rb] = fmaxf(mx[rb], tv[tb][rb]);
            }
        }
        if (a.scores) {
            // (at G = 8 the lane index is recomputed here rather than held for this path)
            const int sl = TBMAJ ? lane_here() : lane, sn = sl & 15, sg4 = sl >> 4;
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    if (tv[tb][rb] != -INFINITY)
                        a.scores[(static_cast<size_t>(b) * a.hq + hq0 + 4 * rb + sg4) * a.capacity + t0 + 16 * tb + sn] =
                            tv[tb][rb] * kLn2;
        }
        bool grow = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) grow = grow || mx[rb] > m_run[rb] + slack;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float mn = fmaxf(m_run[rb], row16_max(mx[rb]));
                const float alpha = mn == m_run[rb] ? 1.0f : __builtin_amdgcn_exp2f(m_run[rb] - mn);
                l_run[rb] *= alpha;
#pragma unroll
                for (int Q = 0; Q < 4; ++Q) acc[rb][Q] *= alpha;
                m_run[rb] = mn;
            }
        }
        float wts[NTB][RB];
        bool keep = false;
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            // rows past the sequence end hold whatever the cache held: weight exactly 0
            const float nvn = 16 * tb + nt < nv ? (V3 ? 1.0f : half_bits_to_float(vt.norm[tb][0])) : 0.0f;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float p = __builtin_amdgcn_exp2f(tv[tb][rb] - m_run[rb]);
                l_run[rb] += p;
                wts[tb][rb] = (p >= a.v_skip ? p : 0.0f) * nvn;
                keep = keep || wts[tb][rb] != 0.0f;
            }
        }
        // the value products of the tile only where some weight is left (uniform); the
        // kernels that load values into registers keep one path (the branch costs them
        // registers)
        if (!VLDS || __builtin_amdgcn_ballot_w64(keep) != 0) {
            // passes of WTB token blocks: their weights to LDS, then their value products (a
            // pass rewrites the weight words only after the previous pass has read them)
            static_for<NTB / WTB>([&](auto pc2) {
                constexpr int TB0 = decltype(pc2)::value * WTB;
                if constexpr (TB0 > 0) lds_order();
                if constexpr (STAGED && WTB < NTB) read_vwords(TB0);
#pragma unroll
                for (int sl = 0; sl < WTB; ++sl) {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                        for (int i = 0; i < (V3 ? 4 : 1); ++i) {  // PQ3: the weight times the norm of block i
                            const int tb = TB0 + sl;
                            const float wt = V3 ? wts[tb][rb] * half_bits_to_float((vnorm[i] >> (16 * tb)) & 0xFFFFu)
                                                : wts[tb][rb];
                            const uint32_t bits = __float_as_uint(wt);
                            const float lo = wt - __uint_as_float(bits & 0xFFFF0000u);
                            uint32_t* dst = wa + w_lane + (i * C::WA + (sl * G + 4 * rb) * 32);
                            dst[0] = dup_hi16(bits);
                            dst[16] = dup_hi16(__float_as_uint(lo));
                        }
                    }
                }
                lds_order();

                // ---- values: job J = sl * 4 + Q reads byte Q of code word n of tokens
                // 16 (TB0 + sl) + 4g .. +3
                // A operands: PQ4 one per token block, read here; PQ3 one per (token block,
                // block of 32), read with the lookups of their job into a ring
                u32x4 av[V3 ? R : WTB][RB];
                auto read_a = [&](u32x4 (&dst)[RB], int i, int sl) __attribute__((always_inline)) {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        dst[rb] = *reinterpret_cast<const u32x4*>(wa + rd_lane + (i * C::WA + (sl * G + 4 * rb) * 32));
                };
                if constexpr (!V3) {
#pragma unroll
                    for (int sl = 0; sl < WTB; ++sl) read_a(av[sl], 0, sl);
                }
                constexpr int NJ = 4 * WTB;
                u32x8 ring[R];
                static_for<NJ + LA>([&](auto jc) {
                    constexpr int J = decltype(jc)::value;
                    if constexpr (J < NJ) {
                        constexpr int SL = J / 4, Q = J % 4;
                        if constexpr (V3) read_a(av[J % R], Q, SL);
#pragma unroll
                        for (int u = 0; u < 4; ++u) put_byte1<Q>(addr[u], vt.w[TB0 + SL][0][u]);
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const uint2 v = *reinterpret_cast<const uint2*>(vtab + addr[u]);
                            ring[J % R][2 * u] = v.x;
                            ring[J % R][2 * u + 1] = v.y;
                        }
                    }
                    if constexpr (J >= LA) {
                        constexpr int M = J - LA, SL = M / 4, Q = M % 4;
                        const bf16x16 bop = __builtin_bit_cast(bf16x16, ring[M % R]);
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb)
                            acc[rb][Q] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(
                                __builtin_bit_cast(bf16x8, av[V3 ? M % R : SL][rb]), bop, acc[rb][Q], sp_idx, 0, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
            });
            lds_order();
        }
        if constexpr (!VLDS) load_values<VBV>(vt, vrn, v_norm, v_word, t_next * VBV);
    };
    if constexpr (VLDS) {
        // pairs of tiles, so that the parity is static; the second tile of the last pair may be
        // empty (its weights are all zero, and the running maximum is finite by then)
        for (; t0 < end; t0 += 2 * kStep) {
            tile(std::integral_constant<int, 0>{}, t0);
            tile(std::integral_constant<int, 1>{}, t0 + kStep);
        }
        // the last requests (tiles past the end) land before the LDS is released
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    } else {
        for (; t0 < end; t0 += kStep) tile(std::integral_constant<int, 0>{}, t0);
    }

    // ---- merge the four wavefronts of each split and write its record
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) l_run[rb] = row16_sum(l_run[rb]);

    __syncthreads();  // every lookup of the workgroup is done: the table area becomes the merge buffer
    float* red = sm.u.red;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float* r = red + (wi * G + 4 * rb + g) * (2 + D);
        if (n == 0) {
            r[0] = m_run[rb];
            r[1] = l_run[rb];
        }
#pragma unroll
        for (int Q = 0; Q < 4; ++Q)
#pragma unroll
            for (int p = 0; p < 2; ++p)  // coordinate 2m + p of pair m: PQ4 byte Q of word n, PQ3 pair n of block Q
                r[2 + (V3 ? 32 * Q + 2 * n : 8 * n + 2 * Q) + p] = acc[rb][Q][p] + acc[rb][Q][2 + p];
    }
    __syncthreads();
    // per split group: the factors of its wavefronts once per (wavefront, head), then the
    // coordinates (the arithmetic and order of merge_factors / merged_coordinate)
    __shared__ float fw_sp[kPairSub][kWaves * G];
    const float* red_sg = red + sg * kWaves * G * (2 + D);
    const int tsg = tid % (kWaves * 64);
    const size_t rec0 = (static_cast<size_t>(b) * a.hq + hq0) * a.splits + s;
    if (s < a.splits && tsg < G) {
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, red_sg[(ww * G + tsg) * (2 + D)]);
        float L = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float* r = red_sg + (ww * G + tsg) * (2 + D);
            const float f = r[0] == -INFINITY ? 0.0f : exp2f(r[0] - M);
            fw_sp[sg][ww * G + tsg] = f;
            L = fmaf(r[1], f, L);
        }
        store_dev(a.ml + rec0 + static_cast<size_t>(tsg) * a.splits, make_float2(M, L));  // device scope: another XCD may merge them
    }
    __syncthreads();
    if (s < a.splits) {
        for (int idx = tsg; idx < G * D; idx += kWaves * 64) {
            const int gg = idx / D, j = idx % D;
            const size_t rec = rec0 + static_cast<size_t>(gg) * a.splits;
            store_dev(a.acc + rec * D + j, merged_coordinate<D, G, kWaves>(red_sg, fw_sp[sg], gg, j));
        }
    }
    // the merge reuses the table and reduction area (the barrier in stream_arrive orders it
    // after the reads of red above)
    constexpr int NT = kPairWaves * 64;
    static_assert(sizeof(sm.u) >= sizeof(float) * (4 * NT + (2 * (NT / G / (D / 4)) + D + 1) * G),
                  "merge buffers fit the reused area");
    stream_finish<D, G, NT>(a, cbv, true, b, h, reinterpret_cast<float*>(&sm.u), &tail_flag);
}

// ---------------------------------------------------------------------------
// TQ3K keys ([P2] trick 2: 2-bit MSE code plus 1-bit QJL sign per coordinate) with
// GQ2V or GQ4V values ([P2] trick 3: v * scale + zero per group), d = 128, up to
// eight query heads per KV head, on the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  Rows of every product are
// (head h, half r of the hi/lo split of the query side), 16 rows for eight heads.
//
// Scores, columns = 16 tokens:
//   MSE  D[(h,r)][t] += sum_{j,s} q_r[h][j] c_s[code_tj]: a lane's eight k are the
//        four coordinates of one code byte with both centroid halves, read as one
//        16-byte entry of a 256-entry LDS table (byte -> (c_hi, c_lo) x 4);
//   QJL  D[(h,r)][t] += sum_j u_r[h][j] (2 b_tj - 1): a lane's eight k are one byte
//        of sign bits, read from a 256-entry table of +-1 octets.
//   The score is n_t (mse + gamma_t qjl) with log2(e)/sqrt(d) folded into both query
//   operands and sqrt(pi/2)/d into the sketch's.  Each table has eight copies, one per
//   lane of an eight-lane LDS phase, so that any bytes read conflict-free.
// Values, per group gr of 32 channels, columns = 16 channels 32 gr + 2 col + hf for
// the two products hf = 0, 1 (one code dword per token serves both):
//   D[(h,r)][col] += sum_t w_r[h][t] (128 + q_tj) with w = p * scale_t,gr split hi/lo;
//   the codes enter exactly as bf16(128 + q) = 0x4300 | q, two tokens per dword by one
//   byte permute, a shift and a mask; then
//   acc_hj = D_hi + D_lo - 128 sum_t (w_hi + w_lo) + sum_t p zero_t,gr,
//   the two sums kept on the VALU by the lanes that own the token's weight.
// Eight wavefronts per workgroup share the tables; each walks 32-token tiles of the
// split with the next tile's keys (registers) and values (an LDS stage, by buffer
// loads with an LDS destination) requested before the current tile's products.
template <int VF>
struct TqCfg {
    static constexpr int D = 128, VBK = 52;
    static constexpr int VBV = VF == TQ_FMT_GQ2V ? 48 : 80;  // value bytes per token
    static constexpr int GB = VF == TQ_FMT_GQ2V ? 12 : 20;   // bytes per value group
    static constexpr int QB = VF == TQ_FMT_GQ2V ? 2 : 4;     // code bits
    static constexpr int WAVES = 8, TT = 32, NTB = TT / 16, NGRP = 4, COPIES = 8;
    static constexpr int STAGE = TT * VBV;                   // a multiple of 256
    // a weight row holds TT tokens and 8 spare entries: rows 80 bytes apart put the eight
    // lanes of an LDS phase of the A-operand reads on distinct banks
    static constexpr int TTP = TT + 8;
};

template <int VF>
struct SmemTq {
    using C = TqCfg<VF>;
    union {
        // both tables in 256-byte rows: row b holds the MSE entry of byte b in its eight copies,
        // then the QJL entry in its eight copies, so that a lookup address is one byte permute
        // of the code word (b << 8 | table << 7 | copy << 4)
        u32x4 tab[256 * 2 * C::COPIES];
        float red[C::WAVES * 8 * (2 + C::D)];  // per-wavefront (m, l, acc) after the tile loop
    } u;
    alignas(16) uint16_t wa[C::WAVES][C::NGRP][16][C::TTP];  // value A operands [group][row][token slot]
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Key bytes of a 16-token block for lane (n, g): token n's norms (n | gamma << 16),
// code bytes 8g .. 8g+7 (coordinates 32g .. 32g+31) and sign byte group g (dword g of
// the QJL bits: coordinates 32g .. 32g+31).
struct TqKeys {
    uint32_t norms[2];
    u32x2 codes[2];
    uint32_t signs[2];
};

__device__ __forceinline__ void load_tq_keys(TqKeys& k, __amdgpu_buffer_rsrc_t r, int lane_off, int g, int tile_off) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int o = lane_off + 16 * tb * 52;
        k.norms[tb] = __builtin_amdgcn_raw_buffer_load_b32(r, o, tile_off, kStreamPolicy);
        k.codes[tb] = __builtin_amdgcn_raw_buffer_load_b64(r, o + 4 + 8 * g, tile_off, kStreamPolicy);
        k.signs[tb] = __builtin_amdgcn_raw_buffer_load_b32(r, o + 36 + 4 * g, tile_off, kStreamPolicy);
    }
}

// bf16 (hi, lo) halves of x as (lo << 16) | hi, by the hardware round-to-nearest-even
// conversion: hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ uint32_t bf16_split_hw(float x) {
    const __bf16 hi = static_cast<__bf16>(x);
    const __bf16 lo = static_cast<__bf16>(x - static_cast<float>(hi));
    uint16_t hb, lb;
    __builtin_memcpy(&hb, &hi, 2);
    __builtin_memcpy(&lb, &lo, 2);
    return hb | (static_cast<uint32_t>(lb) << 16);
}

template <int VF, int G>
__global__ __launch_bounds__(TqCfg<VF>::WAVES * 64) void decode_partial_tq3k_kernel(DecodeArgs a, DevCodebook cbk,
                                                                                      DevCodebook cbv) {
    using C = TqCfg<VF>;
    static_assert(G <= 8, "eight heads fill the sixteen rows");
    constexpr int D = C::D, VBK = C::VBK, VBV = C::VBV, GB = C::GB, TT = C::TT, NW = C::WAVES;
    __shared__ __align__(16) SmemTq<VF> sm;
    __shared__ __align__(16) uint8_t vst0[NW][C::STAGE];
    __shared__ __align__(16) uint8_t vst1[NW][C::STAGE];

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: tile offsets stay in SGPRs
    const int n = lane & 15, g = lane >> 4;
    const int hq0 = h * G;
    const int start = s * a.split_len;
    const size_t rec0 = (static_cast<size_t>(b) * a.hq + hq0) * a.splits + s;

    // ---- the small global reads first: the query entries of the operands this thread builds.
    // Operand entry (job, lane l): jobs 0..7 are the MSE products I, whose lane (row i, group gg)
    // holds coordinates 32 gg + 4 I .. + 3 of head i / 2, half i % 2, each duplicated for the
    // two centroid halves; jobs 8..11 the QJL products I - 8, coordinates 32 gg + 8 (I - 8) .. + 7
    // of the sketch.  768 entries, one or two per thread.
    constexpr int NJOB = 12 * 64;
    float ev[2][8];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int e = tid + NW * 64 * k;
        const int job = (e < NJOB ? e : 0) >> 6, l = e & 63, ri = l & 15, gg = l >> 4;
        const int hh = (ri >> 1) < G ? ri >> 1 : 0;
        const size_t qrow = (static_cast<size_t>(b) * a.hq + hq0 + hh) * D + 32 * gg;
        if (job < 8) {
            const float4 v = *reinterpret_cast<const float4*>(a.q_rot + qrow + 4 * job);
            ev[k][0] = v.x; ev[k][1] = v.y; ev[k][2] = v.z; ev[k][3] = v.w;
            ev[k][4] = ev[k][5] = ev[k][6] = ev[k][7] = 0.0f;
        } else {
            const float4* sp = reinterpret_cast<const float4*>(a.q_sk + qrow + 8 * (job - 8));
            const float4 v0 = sp[0], v1 = sp[1];
            ev[k][0] = v0.x; ev[k][1] = v0.y; ev[k][2] = v0.z; ev[k][3] = v0.w;
            ev[k][4] = v1.x; ev[k][5] = v1.y; ev[k][6] = v1.z; ev[k][7] = v1.w;
        }
    }

    const size_t stream_row = (static_cast<size_t>(b) * a.hkv + h) * a.capacity;
    const __amdgpu_buffer_rsrc_t krs = stream_rsrc(a.k_cache + stream_row * VBK, static_cast<uint32_t>(a.capacity) * VBK);
    const __amdgpu_buffer_rsrc_t vrs = stream_rsrc(a.v_cache + stream_row * VBV, static_cast<uint32_t>(a.capacity) * VBV);
    const __amdgpu_buffer_rsrc_t krs_none = null_rsrc(a.k_cache), vrs_none = null_rsrc(a.v_cache);
    const int k_lane = n * VBK;

    // the first tile of this wavefront, requested before the sequence length arrives: its
    // bytes lie inside the stream's range (the resource returns zeros past it), and a tile
    // at or past the end is read and not used
    constexpr int kStep = NW * TT;
    int t0 = start + w * TT;
    TqKeys kt[2];
    stage_bytes<C::STAGE>(vrs, vst0[w], t0 * VBV, lane);  // values first: the wait for the keys covers them
    load_tq_keys(kt[0], krs, k_lane, g, t0 * VBK);
    __builtin_amdgcn_sched_barrier(0);

    int N = a.seq_lens[b];
    N = N < 0 ? 0 : (N > a.capacity ? a.capacity : N);
    const int end = min(start + a.split_len, N);
    if (start >= end) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the staged tile lands before the LDS is released
        for (int gg = 0; gg < G; ++gg) {
            const size_t rec = rec0 + static_cast<size_t>(gg) * a.splits;
            if (tid == 0) a.ml[rec] = make_float2(-INFINITY, 0.0f);
            for (int j = tid; j < D; j += blockDim.x) a.acc[rec * D + j] = 0.0f;
        }
        return;
    }

    // ---- tables: thread t fills entries t + 512 k (entry e is byte e / COPIES, copy e % COPIES)
    {
        uint32_t csp[4];  // (hi, lo) of the four key centroids
#pragma unroll
        for (int c = 0; c < 4; ++c) csp[c] = bf16_split_hw(cbk.centroids[c]);
#pragma unroll
        for (int k = 0; k < 256 * C::COPIES / (NW * 64); ++k) {
            const int e = tid + NW * 64 * k;
            const uint32_t byte = static_cast<uint32_t>(e) / C::COPIES;
            u32x4 m, q;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t b0 = (byte >> (2 * c)) & 1u, b1 = (byte >> (2 * c + 1)) & 1u;
                m[c] = b1 ? (b0 ? csp[3] : csp[2]) : (b0 ? csp[1] : csp[0]);
                q[c] = (b0 ? 0x3F80u : 0xBF80u) | ((b1 ? 0x3F80u : 0xBF80u) << 16);
            }
            sm.u.tab[(2 * byte) * C::COPIES + (e % C::COPIES)] = m;
            sm.u.tab[(2 * byte + 1) * C::COPIES + (e % C::COPIES)] = q;
        }
    }
    // ---- query operands into LDS (the weight area, free until the first tile): the query times
    // log2(e)/sqrt(d), the sketch also times sqrt(pi/2)/d, as bf16 halves (rows of heads >= G zero)
    u32x4* opl = reinterpret_cast<u32x4*>(&sm.wa[0][0][0][0]);  // [job][lane]
    static_assert(sizeof(sm.wa) >= sizeof(u32x4) * NJOB, "operands fit the weight area");
    {
        const float qscale = kLog2e / sqrtf(static_cast<float>(D));
        const float sscale = qscale * (1.2533141373155003f / D);  // sqrt(pi/2)/d
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = tid + NW * 64 * k;
            if (e < NJOB) {
                const int job = e >> 6, ri = e & 15;
                const bool live = (ri >> 1) < G;
                const uint32_t sh = (ri & 1) * 16;  // half r of the split
                u32x4 v;
                if (job < 8) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint32_t hv = live ? (bf16_split_hw(ev[k][c] * qscale) >> sh) & 0xFFFFu : 0u;
                        v[c] = hv | (hv << 16);
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint32_t h0 = (bf16_split_hw(ev[k][2 * c] * sscale) >> sh) & 0xFFFFu;
                        const uint32_t h1 = (bf16_split_hw(ev[k][2 * c + 1] * sscale) >> sh) & 0xFFFFu;
                        v[c] = live ? h0 | (h1 << 16) : 0u;
                    }
                }
                opl[e] = v;
            }
        }
    }
    lds_write_barrier();  // the first tile stays in flight
    u32x4 qa[8], sa[4];
#pragma unroll
    for (int I = 0; I < 8; ++I) qa[I] = opl[I * 64 + lane];
#pragma unroll
    for (int I = 0; I < 4; ++I) sa[I] = opl[(8 + I) * 64 + lane];
    lds_write_barrier();  // every wavefront holds its operands before any writes weights there

    // per lane: heads 2g + e (rows 4g + 2e + r of every product); rows of heads >= G stay at
    // m = 0, p = 0
    float m_run[2], l_run[2], zacc[2][4];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        m_run[e] = (2 * g + e < G) ? -INFINITY : 0.0f;
        l_run[e] = 0.0f;
#pragma unroll
        for (int gr = 0; gr < 4; ++gr) zacc[e][gr] = 0.0f;
    }
    f32x4 acc[4][2], wsum[4];  // value sums per group and product; sum of the weight halves per group
#pragma unroll
    for (int gr = 0; gr < 4; ++gr) acc[gr][0] = acc[gr][1] = wsum[gr] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const char* tabs = reinterpret_cast<const char*>(sm.u.tab);
    // byte 0 of a lookup address: this lane's copy (lane & 7), and the QJL half of the row
    const uint32_t lc_m = (lane & 7) * 16u, lc_q = lc_m | 128u;
    const float slack = a.v_skip > 0.0f ? 0.0f : kRescaleSlack;
    // this lane's code dword of a group and the byte of it holding channels 2n, 2n + 1
    constexpr int QB = C::QB;
    const int cw_off = QB == 2 ? 4 + 4 * (n >> 3) : 4 + 4 * (n >> 2);
    const uint32_t cbyte = QB == 2 ? (n & 7) >> 1 : (n & 3);
    const uint32_t csh = QB == 2 ? 4 * (n & 1) : 0;  // bit of channel 2n within that byte
    const uint32_t psel = cbyte | (0x0Cu << 8) | ((cbyte + 4u) << 16) | (0x0Cu << 24);
    // Channel 2n + hf of a token's byte pair, as bf16(128 + c q) with q its code: 2-bit codes
    // after one shift by csh, hf = 0 masked in place (c = 1) and hf = 1 two bits up (c = 4, the
    // product scaled back by 1/4 at the end); 4-bit codes the low nibble in place and the high
    // nibble after a shift by 4 (c = 1).  Masks in registers: mask and or fuse into one
    // instruction.
    constexpr uint32_t csh1 = QB == 2 ? 0u : 4u;
    constexpr float kHf1 = QB == 2 ? 0.25f : 1.0f;
    uint32_t cmask0 = QB == 2 ? 0x00030003u : 0x000F000Fu, cmask1 = QB == 2 ? 0x000C000Cu : 0x000F000Fu;
    asm("" : "+v"(cmask0), "+v"(cmask1));
    const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    constexpr int TTP = C::TTP;
    uint16_t* wa_w = &sm.wa[w][0][0][0];
    uint32_t* wa_w32 = reinterpret_cast<uint32_t*>(wa_w);
    // Token slots: token 8 q + j of a tile sits in slot 8 q + ((j - 2 q) & 7) of its weight rows,
    // and the value product's lane group q takes its eight tokens in that order, so that the
    // four lane groups read four different token rows of the stage at any step and the code
    // reads of a step fall on distinct banks.  The rotation is even: a token pair (2i, 2i + 1)
    // keeps two adjacent slots, one dword.
    uint32_t wslot[2];  // dword of this lane's token pair in a weight row, per token block
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int tp = 16 * tb + (n & ~1), q = tp >> 3;
        wslot[tb] = static_cast<uint32_t>(4 * q + ((((tp & 7) - 2 * q) & 7) >> 1));
    }
    // dword of a group pair's even / odd group: the even lane (mine = its H, nb = the odd
    // neighbour's H) takes (mine, nb) halves, the odd lane (mine = its L, nb = the even
    // neighbour's L) takes (nb, mine)
    const uint32_t wsel0 = (n & 1) ? 0x01000504u : 0x05040100u;
    const uint32_t wsel1 = (n & 1) ? 0x03020706u : 0x07060302u;
    const int t_first = start + w * TT;
    uint32_t xoff[8];  // stage offset of the code dword of the u-th token of lane group g
#pragma unroll
    for (int u = 0; u < 8; ++u) xoff[u] = lds_offset((8 * g + ((u + 2 * g) & 7)) * VBV + cw_off);

    auto tile = [&](auto pc, const int t0) {
        constexpr int P = decltype(pc)::value;
        TqKeys& kc = kt[P];
        const int nv = min(TT, end - t0);  // <= 0 for the odd tile after the last one
        const bool more = t0 + kStep < end;
        const int t_next = more ? t0 + kStep : t0;
        const uint8_t* vcur = P == 0 ? vst0[w] : vst1[w];
        stage_bytes<C::STAGE>(more ? vrs : vrs_none, P == 0 ? vst1[w] : vst0[w], t_next * VBV, lane);
        load_tq_keys(kt[1 - P], more ? krs : krs_none, k_lane, g, t_next * VBK);

        // ---- scores: job J is product I = J / 2 of token block J % 2 (I < 8: the MSE products,
        // I = 8 .. 11: the QJL products), so that the two blocks' accumulator chains interleave
        float tv[2][2];
        {
            f32x4 dm[2], dq[2];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) dm[tb] = dq[tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            constexpr int LA = 2, NJ = 24, R = LA + 1;
            u32x4 ring[R];
            static_for<NJ + LA>([&](auto jc) {
                constexpr int J = decltype(jc)::value;
                if constexpr (J < NJ) {
                    constexpr int I = J / 2, TB = J % 2;
                    // address bytes: (lane constant, code byte k, 0, 0)
                    if constexpr (I < 8) {
                        const uint32_t word = I < 4 ? kc.codes[TB][0] : kc.codes[TB][1];
                        const uint32_t ad = __builtin_amdgcn_perm(word, lc_m, 0x0C0C0400u + ((I % 4) << 8));
                        ring[J % R] = *reinterpret_cast<const u32x4*>(tabs + ad);
                    } else {
                        const uint32_t ad = __builtin_amdgcn_perm(kc.signs[TB], lc_q, 0x0C0C0400u + ((I - 8) << 8));
                        ring[J % R] = *reinterpret_cast<const u32x4*>(tabs + ad);
                    }
                }
                if constexpr (J >= LA) {
                    constexpr int M = J - LA, I = M / 2, TB = M % 2;
                    const bf16x8 bop = __builtin_bit_cast(bf16x8, ring[M % R]);
                    if constexpr (I < 8)
                        dm[TB] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[I]), bop, dm[TB],
                                                                         0, 0, 0);
                    else
                        dq[TB] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, sa[I - 8]), bop,
                                                                         dq[TB], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const float nk = half_bits_to_float(kc.norms[tb] & 0xFFFFu);
                const float gk = half_bits_to_float(kc.norms[tb] >> 16);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const bool ok = 2 * g + e < G && 16 * tb + n < nv;
                    const float sc = nk * fmaf(gk, dq[tb][2 * e] + dq[tb][2 * e + 1], dm[tb][2 * e] + dm[tb][2 * e + 1]);
                    tv[tb][e] = ok ? sc : -INFINITY;
                }
            }
        }
        if (a.scores) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    if (tv[tb][e] != -INFINITY)
                        a.scores[(static_cast<size_t>(b) * a.hq + hq0 + 2 * g + e) * a.capacity + t0 + 16 * tb + n] =
                            tv[tb][e] * kLn2;
        }

        // ---- online softmax; lane (n, g) owns token 16 tb + n of heads 2g, 2g + 1
        float mx[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) mx[e] = fmaxf(tv[0][e], tv[1][e]);
        if (__builtin_amdgcn_ballot_w64(mx[0] > m_run[0] + slack || mx[1] > m_run[1] + slack) != 0) {
            // before the wavefront's first tile every sum is zero: only the reference moves
            const bool first = t0 == t_first;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float mn = fmaxf(m_run[e], row16_max(mx[e]));
                if (!first) {
                    const float alpha = mn == m_run[e] ? 1.0f : __builtin_amdgcn_exp2f(m_run[e] - mn);
                    l_run[e] *= alpha;
#pragma unroll
                    for (int gr = 0; gr < 4; ++gr) {
                        zacc[e][gr] *= alpha;
                        wsum[gr][2 * e] *= alpha;
                        wsum[gr][2 * e + 1] *= alpha;
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) {
                            acc[gr][hf][2 * e] *= alpha;
                            acc[gr][hf][2 * e + 1] *= alpha;
                        }
                    }
                }
                m_run[e] = mn;
            }
        }
        // weights times each group's scale, as the A operands of the value products, split into
        // bf16 halves two groups at a time: H = (hi of group 2k, hi of group 2k + 1), L the lo
        // halves.  Lanes n and n ^ 1 hold a token pair: the even lane writes the pair's hi
        // halves (row 4g + 2e), the odd lane the lo halves (row 4g + 2e + 1), one dword per group
        bool keep = false;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int t = 16 * tb + n;
            const bool tok = t < nv;
            uint32_t hdr[4];  // the token's (scale, zero) per group as fp16 pairs (0 past the end: never stale)
#pragma unroll
            for (int gr = 0; gr < 4; ++gr) {
                const uint32_t x = *reinterpret_cast<const uint32_t*>(vcur + lds_offset(t * VBV) + GB * gr);
                hdr[gr] = tok ? x : 0u;
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float p = __builtin_amdgcn_exp2f(tv[tb][e] - m_run[e]);  // 0 for invalid tokens and rows
                l_run[e] += p;
                const float pk = p >= a.v_skip ? p : 0.0f;
                keep = keep || pk != 0.0f;
                uint32_t* dst = wa_w32 + lds_offset((4 * g + 2 * e + (n & 1)) * (TTP / 2) + wslot[tb]);
#pragma unroll
                for (int gp = 0; gp < 2; ++gp) {
                    float wv[2];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int gr = 2 * gp + i;
                        zacc[e][gr] = fmaf(pk, half_bits_to_float(hdr[gr] >> 16), zacc[e][gr]);
                        wv[i] = pk * half_bits_to_float(hdr[gr] & 0xFFFFu);
                    }
                    const uint32_t H = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{wv[0], wv[1]}, bf16x2_t));
                    const float r0 = wv[0] - __uint_as_float(H << 16), r1 = wv[1] - __uint_as_float(H & 0xFFFF0000u);
                    const uint32_t Lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{r0, r1}, bf16x2_t));
                    const uint32_t mine = (n & 1) ? Lo : H, give = (n & 1) ? H : Lo;
                    const uint32_t nb = static_cast<uint32_t>(
                        __builtin_amdgcn_mov_dpp(static_cast<int>(give), kDppXor1, 0xF, 0xF, false));
                    dst[(2 * gp) * 16 * (TTP / 2)] = __builtin_amdgcn_perm(nb, mine, wsel0);
                    dst[(2 * gp + 1) * 16 * (TTP / 2)] = __builtin_amdgcn_perm(nb, mine, wsel1);
                }
            }
        }
        if (__builtin_amdgcn_ballot_w64(keep) == 0) return;  // no value survives (uniform)
        lds_order();

        // ---- values: per group, the A operand (rows, tokens 8g .. 8g+7) and the code dwords
        // of those tokens; product hf takes channels 32 gr + 2 col + hf, and a product with a
        // B of ones sums the weight halves the value products used
#pragma unroll
        for (int gr = 0; gr < 4; ++gr) {
            const u32x4 av = *reinterpret_cast<const u32x4*>(wa_w + lds_offset((gr * 16 + n) * TTP + 8 * g));
            uint32_t x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const uint32_t*>(vcur + xoff[u] + GB * gr);
            uint32_t pr[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) pr[v] = __builtin_amdgcn_perm(x[2 * v + 1], x[2 * v], psel);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                u32x4 bv;
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    bv[v] = hf == 0 ? ((pr[v] >> csh) & cmask0) | 0x43004300u
                                    : ((pr[v] >> (csh + csh1)) & cmask1) | 0x43004300u;
                acc[gr][hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                                      __builtin_bit_cast(bf16x8, bv), acc[gr][hf], 0, 0, 0);
            }
            wsum[gr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                               __builtin_bit_cast(bf16x8, ones), wsum[gr], 0, 0, 0);
        }
        lds_order();
    };
    for (; t0 < end; t0 += 2 * kStep) {
        tile(std::integral_constant<int, 0>{}, t0);
        tile(std::integral_constant<int, 1>{}, t0 + kStep);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the last requests land before the LDS is released

    // ---- the zero terms summed over the 16 token lanes, then the wavefronts merge
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        l_run[e] = row16_sum(l_run[e]);
#pragma unroll
        for (int gr = 0; gr < 4; ++gr) zacc[e][gr] = row16_sum(zacc[e][gr]);
    }
    __syncthreads();  // every table lookup of the workgroup is done: the tables become the merge buffer
    float* red = sm.u.red;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int hh = 2 * g + e;
        if (hh < G) {
            float* r = red + (w * G + hh) * (2 + D);
            if (n == 0) {
                r[0] = m_run[e];
                r[1] = l_run[e];
            }
#pragma unroll
            for (int gr = 0; gr < 4; ++gr) {
                const float corr = 128.0f * (wsum[gr][2 * e] + wsum[gr][2 * e + 1]);
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    r[2 + 32 * gr + 2 * n + hf] =
                        ((acc[gr][hf][2 * e] + acc[gr][hf][2 * e + 1]) - corr) * (hf ? kHf1 : 1.0f) + zacc[e][gr];
            }
        }
    }
    __syncthreads();
    __shared__ float fw[NW * G];
    merge_factors<D, G, NW>(red, fw, tid, a.ml + rec0, a.splits);
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += blockDim.x) {
        const int gg = idx / D, j = idx % D;
        const size_t rec = rec0 + static_cast<size_t>(gg) * a.splits;
        a.acc[rec * D + j] = merged_coordinate<D, G, NW>(red, fw, gg, j);
    }
}

int auto_split_tokens(const tq_layout* L) {
    const long streams = static_cast<long>(L->batch) * L->n_kv_heads;
    const long max_splits = (L->capacity + kSplitQuantum - 1) / kSplitQuantum;
    // Splits per launch, measured per kernel:
    //   * PQ4 at d = 128, G = 4 or 8 (2:4-sparse kernel): four splits per 16-wavefront workgroup,
    //     one workgroup per CU, so about 1024 splits fill the chip in a single round;
    //   * PQ4 at d = 256, G = 4 or 8: one split per 8-wavefront workgroup of the byte-pair kernel
    //     (150 KB of LDS), one workgroup per CU, about 256 splits; the dense bf16 kernel
    //     (distinct key and value centroids) runs the same splits at two 4-wavefront
    //     workgroups per CU (c5: 44 us at 512 splits with it, 47 at 256, 62 at 2048);
    //   * the generic kernel: about 2048 splits, two rounds of four workgroups per CU.
    //   * TQ3K keys at d = 128 (matrix-core kernel, eight wavefronts and 136 KB of LDS per
    //     workgroup): one workgroup per CU, about 256 splits;
    const int G = L->n_kv_heads > 0 ? L->n_q_heads / L->n_kv_heads : 0;
    //   * PQ3 keys at d = 128, G = 4 (the 2:4-sparse kernel too): as PQ4.
    const bool pq4 = L->k_format == TQ_FMT_PQ4 && L->v_format == TQ_FMT_PQ4 && (G == 4 || G == 8);
    const bool pq3 = L->k_format == TQ_FMT_PQ3 && L->head_dim == 128 && G == 4;
    const bool tq3k = L->k_format == TQ_FMT_TQ3K && L->head_dim == 128 && G <= 8;
    const long target = pq4 ? (L->head_dim == 128 ? 1024 : 256) : pq3 ? 1024 : tq3k ? 256 : 2048;
    long want = (target + streams - 1) / streams;
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

// Stream of a decode launch, and optionally events that the runtime attaches to
// the kernel's own dispatch (start and end of the kernel itself).
struct Launch {
    hipStream_t st;
    hipEvent_t start, stop;
};

template <typename K, typename... Args>
int launch_kernel(K kernel, dim3 grid, dim3 block, const Launch& l, Args... args) {
    if (l.start || l.stop)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, l.st, l.start, l.stop, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, l.st, args...);
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

template <int KF, int VF, int D, int G>
int launch_partial(const DecodeArgs& a, const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv,
                   const Launch& l) {
    dim3 grid(a.splits, L->n_kv_heads, L->batch);
    return launch_kernel(decode_partial_kernel<KF, VF, D, G>, grid, dim3(kWaves * 64), l, a, to_dev(cbk), to_dev(cbv));
}

// tokens per wavefront tile of the bf16 decode kernel (16 or a multiple of 16 dividing 64)
constexpr int kBf16Tile = 32;

template <int G, bool VTAB, int KF = TQ_FMT_PQ4, int VF = TQ_FMT_PQ4>
int launch_partial_sparse(const DecodeArgs& a, const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv,
                          const Launch& l) {
    dim3 grid((a.splits + kPairSub - 1) / kPairSub, L->n_kv_heads, L->batch);
    return launch_kernel(decode_partial_sparse_kernel<G, VTAB, KF, VF>, grid, dim3(kPairWaves * 64), l, a,
                         to_dev(cbk), to_dev(cbv));
}

// K and V decode through one table only when their centroids are identical
bool same_centroids(const tq_codebook& x, const tq_codebook& y) {
    if (x.n_levels != y.n_levels) return false;
    for (int k = 0; k < x.n_levels; ++k)
        if (x.centroids[k] != y.centroids[k]) return false;
    return true;
}

// The kernel that rotates an unrotated query in its prologue: PQ4 keys and values at d 128,
// four query heads per KV head, one centroid table (the values staged through LDS).
bool rotates_in_kernel(const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv) {
    return L->k_format == TQ_FMT_PQ4 && L->v_format == TQ_FMT_PQ4 && L->head_dim == 128 &&
           L->n_q_heads == 4 * L->n_kv_heads && static_cast<size_t>(L->capacity) * 68 <= 0x7FFFFFFFu &&
           same_centroids(cbk, cbv);
}

// The layouts that decode on the 2:4-sparse kernel (which also merges a stream's records
// itself when given an output): d 128 with PQ4 keys and values at G = 4, or at G = 8 with
// one table; PQ3 keys with PQ3 values of the same table, or with PQ4 values, at G = 4.
// dispatch_group launches it exactly for these.
bool sparse_kernel_serves(const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv) {
    if (L->head_dim != 128) return false;
    const int kf = L->k_format, vf = L->v_format, G = L->n_q_heads / L->n_kv_heads;
    const size_t row = std::max(tq::vector_bytes(kf, 128), tq::vector_bytes(vf, 128));
    if (static_cast<size_t>(L->capacity) * row > 0x7FFFFFFFu) return false;  // 32-bit buffer ranges
    if (kf == TQ_FMT_PQ4 && vf == TQ_FMT_PQ4) return G == 4 || (G == 8 && same_centroids(cbk, cbv));
    if (kf == TQ_FMT_PQ3 && vf == TQ_FMT_PQ3) return G == 4 && same_centroids(cbk, cbv);
    if (kf == TQ_FMT_PQ3 && vf == TQ_FMT_PQ4) return G == 4;
    return false;
}

bool merges_in_kernel(const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv) {
    return sparse_kernel_serves(L, cbk, cbv);
}

template <int D, int G>
int launch_partial_bf16(const DecodeArgs& a, const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv,
                        const Launch& l) {
    dim3 grid(a.splits, L->n_kv_heads, L->batch);
    return launch_kernel(decode_partial_bf16_kernel<D, G, kBf16Tile>, grid, dim3(kWaves * 64), l, a, to_dev(cbk),
                         to_dev(cbv));
}

template <int G>
int launch_partial_d256(const DecodeArgs& a, const tq_layout* L, const tq_codebook& cbk, const Launch& l) {
    dim3 grid(a.splits, L->n_kv_heads, L->batch);
    return launch_kernel(decode_partial_d256_kernel<G>, grid, dim3(D256Cfg<G>::NW * 64), l, a, to_dev(cbk));
}

template <int VF, int G>
int launch_partial_tq3k(const DecodeArgs& a, const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv,
                        const Launch& l) {
    dim3 grid(a.splits, L->n_kv_heads, L->batch);
    return launch_kernel(decode_partial_tq3k_kernel<VF, G>, grid, dim3(TqCfg<VF>::WAVES * 64), l, a, to_dev(cbk),
                         to_dev(cbv));
}

template <int KF, int VF, int D>
int dispatch_group(int G, const DecodeArgs& a, const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv,
                   const Launch& st) {
    if constexpr (KF == TQ_FMT_TQ3K && D == 128) {
        // the matrix-core kernel reads the query operands as 16-byte vectors and addresses a
        // stream through a 32-bit buffer range
        const bool ok = aligned(a.q_rot, 16) && aligned(a.q_sk, 16) &&
                        static_cast<size_t>(L->capacity) * vbytes<VF, D>() <= 0x7FFFFFFFu;
        if (ok) {
            switch (G) {
                case 1: return launch_partial_tq3k<VF, 1>(a, L, cbk, cbv, st);
                case 2: return launch_partial_tq3k<VF, 2>(a, L, cbk, cbv, st);
                case 4: return launch_partial_tq3k<VF, 4>(a, L, cbk, cbv, st);
                case 5: return launch_partial_tq3k<VF, 5>(a, L, cbk, cbv, st);
                case 8: return launch_partial_tq3k<VF, 8>(a, L, cbk, cbv, st);
                default: break;
            }
        }
    }
    if constexpr (D == 128 && KF == TQ_FMT_PQ3) {
        if (sparse_kernel_serves(L, cbk, cbv)) {
            if constexpr (VF == TQ_FMT_PQ3) return launch_partial_sparse<4, false, KF, VF>(a, L, cbk, cbv, st);
            else if constexpr (VF == TQ_FMT_PQ4) return launch_partial_sparse<4, true, KF, VF>(a, L, cbk, cbv, st);
        }
    }
    if constexpr (KF == TQ_FMT_PQ4 && VF == TQ_FMT_PQ4) {
        // the matrix-core kernel addresses a stream through a 32-bit buffer range
        const bool fits = static_cast<size_t>(L->capacity) * vbytes<TQ_FMT_PQ4, D>() <= 0x7FFFFFFFu;
        if constexpr (D == 128) {
            if (sparse_kernel_serves(L, cbk, cbv)) {
                if (G == 4) return same_centroids(cbk, cbv) ? launch_partial_sparse<4, false>(a, L, cbk, cbv, st)
                                                            : launch_partial_sparse<4, true>(a, L, cbk, cbv, st);
                return launch_partial_sparse<8, false>(a, L, cbk, cbv, st);
            }
        }
        if constexpr (D == 256) {
            // one table for keys and values: the byte-pair kernel
            if (fits && same_centroids(cbk, cbv)) {
                if (G == 4) return launch_partial_d256<4>(a, L, cbk, st);
                if (G == 8) return launch_partial_d256<8>(a, L, cbk, st);
            }
        }
        if (fits && G == 4) return launch_partial_bf16<D, 4>(a, L, cbk, cbv, st);
        if (fits && G == 8) return launch_partial_bf16<D, 8>(a, L, cbk, cbv, st);
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
                 const Launch& st) {
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

// Workspace of `splits` records per (b, query head) row.
size_t workspace_bytes(const tq_layout* L, int split_tokens) {
    if (check_layout(L) != TQ_OK) return 0;
    int len = 0;
    const int splits = resolve_splits(L, split_tokens, &len);
    if (splits <= 0) return 0;
    return ws_layout(*L, splits).total;
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
    return tq::workspace_bytes(L, split_tokens);
}

size_t tq_decode_hybrid_workspace_bytes(const tq_layout* L, int split_tokens) {
    return tq::workspace_bytes(L, split_tokens);  // the ring is merged in the combine: no record of its own
}

int tq_decode_workspace_init(const tq_layout* L, int split_tokens, void* ws, size_t ws_bytes, hipStream_t stream) {
    using namespace tq;
    const int st = check_layout(L);
    if (st != TQ_OK) return st;
    int len = 0;
    const int splits = resolve_splits(L, split_tokens, &len);
    if (splits <= 0 || !ws || !aligned(ws, 16)) return TQ_ERR_INVALID;
    const WsLayout wl = ws_layout(*L, splits);
    if (ws_bytes < wl.total) return TQ_ERR_WORKSPACE;
    return clear_words(reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + wl.cnt),
                       static_cast<size_t>(L->batch) * L->n_kv_heads, stream);
}

}  // extern "C"

namespace tq {
namespace {

// Checks every argument of a partial call and fills its kernel arguments; nothing is launched.
int partial_args(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const float* q_rot,
                 const float* q_sketch, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                 float* scores, int split_tokens, void* ws, size_t ws_bytes, float v_skip, DecodeArgs* a) {
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
    if (!(v_skip >= 0.0f && v_skip <= 1.0f)) return TQ_ERR_INVALID;  // NaN fails too
    if (ws_bytes < workspace_bytes(L, split_tokens)) return TQ_ERR_WORKSPACE;
    *a = DecodeArgs{};
    a->q_rot = q_rot;
    a->q_sk = q_sketch;
    a->k_cache = static_cast<const uint8_t*>(k_cache);
    a->v_cache = static_cast<const uint8_t*>(v_cache);
    a->seq_lens = seq_lens;
    a->scores = scores;
    const WsLayout wl = ws_layout(*L, splits);
    a->ml = static_cast<float2*>(ws);
    a->acc = reinterpret_cast<float*>(static_cast<char*>(ws) + wl.acc);
    a->arrivals = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + wl.cnt);
    a->hq = L->n_q_heads;
    a->hkv = L->n_kv_heads;
    a->capacity = L->capacity;
    a->splits = splits;
    a->split_len = len;
    a->v_skip = v_skip;
    return TQ_OK;
}

int dispatch_partial(const DecodeArgs& a, const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv,
                     const Launch& stream) {
    const int kf = L->k_format, vf = L->v_format;
    if (kf == TQ_FMT_PQ4 && vf == TQ_FMT_PQ4) return dispatch_dim<TQ_FMT_PQ4, TQ_FMT_PQ4>(a, L, cbk, cbv, stream);
    if (kf == TQ_FMT_PQ3 && vf == TQ_FMT_PQ3) return dispatch_dim<TQ_FMT_PQ3, TQ_FMT_PQ3>(a, L, cbk, cbv, stream);
    if (kf == TQ_FMT_PQ3 && vf == TQ_FMT_PQ4) return dispatch_dim<TQ_FMT_PQ3, TQ_FMT_PQ4>(a, L, cbk, cbv, stream);
    if (kf == TQ_FMT_TQ3K && vf == TQ_FMT_GQ2V) return dispatch_dim<TQ_FMT_TQ3K, TQ_FMT_GQ2V>(a, L, cbk, cbv, stream);
    if (kf == TQ_FMT_TQ3K && vf == TQ_FMT_GQ4V) return dispatch_dim<TQ_FMT_TQ3K, TQ_FMT_GQ4V>(a, L, cbk, cbv, stream);
    return TQ_ERR_UNSUPPORTED;
}

// One partial launch, and the output when `out` is set: merged by the partial kernel's
// last workgroup per stream where it can (one launch), else by the combine kernel after it.
int run_partial(DecodeArgs a, const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv, const Launch& l,
                float* out) {
    if (out && merges_in_kernel(L, cbk, cbv)) {
        a.out = out;
        return dispatch_partial(a, L, cbk, cbv, l);
    }
    const int st = dispatch_partial(a, L, cbk, cbv, l);
    if (st != TQ_OK || !out) return st;
    return combine(L, nullptr, cbv, a.splits, a.ml, out, l.st);
}

// Split records of the compressed cache (and the output when `out` is set).
int decode_partial(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const float* q_rot,
                   const float* q_sketch, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                   float* scores, int split_tokens, void* ws, size_t ws_bytes, const Launch& stream,
                   float v_skip = 0.0f, float* out = nullptr) {
    DecodeArgs a;
    const int st = partial_args(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, seq_lens, scores, split_tokens, ws,
                                ws_bytes, v_skip, &a);
    return st != TQ_OK ? st : run_partial(a, L, *cbk, *cbv, stream, out);
}

}  // namespace
}  // namespace tq

extern "C" {

int tq_decode_partial(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const float* q_rot,
                      const float* q_sketch, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                      float* scores, int split_tokens, void* ws, size_t ws_bytes, hipStream_t stream) {
    return tq::decode_partial(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, seq_lens, scores, split_tokens, ws,
                              ws_bytes, tq::Launch{stream, nullptr, nullptr});
}

int tq_decode_partial_timed(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const float* q_rot,
                            const float* q_sketch, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                            float* scores, int split_tokens, void* ws, size_t ws_bytes, hipStream_t stream,
                            hipEvent_t start, hipEvent_t stop) {
    if (!start || !stop) return TQ_ERR_INVALID;
    return tq::decode_partial(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, seq_lens, scores, split_tokens, ws,
                              ws_bytes, tq::Launch{stream, start, stop});
}

int tq_decode_partial_from_query(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const float* q,
                                 float* q_rot_scratch, const void* k_cache, const void* v_cache,
                                 const int32_t* seq_lens, float* scores, int split_tokens, void* ws, size_t ws_bytes,
                                 hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    using namespace tq;
    if (!L || L->k_format == TQ_FMT_TQ3K) return L ? TQ_ERR_UNSUPPORTED : TQ_ERR_INVALID;  // TQ3K needs the sketch
    if (!q || !aligned(q, 16) || !aligned(q_rot_scratch, 16) || (start == nullptr) != (stop == nullptr))
        return TQ_ERR_INVALID;
    DecodeArgs a;
    const int st = partial_args(L, cbk, cbv, q_rot_scratch, nullptr, k_cache, v_cache, seq_lens, scores,
                                split_tokens, ws, ws_bytes, 0.0f, &a);
    if (st != TQ_OK) return st;
    const Launch l{stream, start, stop};
    if (rotates_in_kernel(L, *cbk, *cbv)) {
        a.q_raw = q;  // rotated in the kernel's prologue; the scratch stays untouched
        return dispatch_partial(a, L, *cbk, *cbv, l);
    }
    const int rs = tq_rotate_sketch_query(L, cbk, nullptr, q, q_rot_scratch, nullptr, stream);
    return rs != TQ_OK ? rs : dispatch_partial(a, L, *cbk, *cbv, l);
}

int tq_decode_step(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const void* k_new,
                   const void* v_new, const int32_t* new_pos, const float* q, float* q_rot_scratch, void* k_cache,
                   void* v_cache, const int32_t* seq_lens, float* out, float* scores, int split_tokens, void* ws,
                   size_t ws_bytes, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    using namespace tq;
    if (!L || L->k_format == TQ_FMT_TQ3K) return L ? TQ_ERR_UNSUPPORTED : TQ_ERR_INVALID;  // TQ3K needs S
    if (!q || !aligned(q, 16) || !aligned(q_rot_scratch, 16) || (start == nullptr) != (stop == nullptr))
        return TQ_ERR_INVALID;
    if (out && !aligned(out, 4)) return TQ_ERR_INVALID;
    if (!k_new || !v_new || !new_pos || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(new_pos, 4))
        return TQ_ERR_INVALID;
    DecodeArgs a;
    int st = partial_args(L, cbk, cbv, q_rot_scratch, nullptr, k_cache, v_cache, seq_lens, scores, split_tokens, ws,
                          ws_bytes, 0.0f, &a);
    if (st != TQ_OK) return st;
    const Launch l{stream, start, stop};
    if (rotates_in_kernel(L, *cbk, *cbv)) {  // one launch: append, rotation and partial
        a.q_raw = q;
        a.k_new = static_cast<const uint16_t*>(k_new);
        a.v_new = static_cast<const uint16_t*>(v_new);
        a.new_pos = new_pos;
        a.k_wr = static_cast<uint8_t*>(k_cache);
        a.v_wr = static_cast<uint8_t*>(v_cache);
        return run_partial(a, L, *cbk, *cbv, l, out);
    }
    // the new rows as a ring of one slot per stream, flushed at new_pos; then the rotation
    st = tq_ring_flush(L, cbk, cbv, nullptr, 1, k_new, v_new, new_pos, 1, k_cache, v_cache, stream);
    if (st != TQ_OK) return st;
    st = tq_rotate_sketch_query(L, cbk, nullptr, q, q_rot_scratch, nullptr, stream);
    return st != TQ_OK ? st : run_partial(a, L, *cbk, *cbv, l, out);
}

int tq_decode_partial_sparse_v(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const float* q_rot,
                               const float* q_sketch, const void* k_cache, const void* v_cache,
                               const int32_t* seq_lens, float* scores, int split_tokens, float v_threshold, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
    return tq::decode_partial(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, seq_lens, scores, split_tokens, ws,
                              ws_bytes, tq::Launch{stream, nullptr, nullptr}, v_threshold);
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
    return combine(L, nullptr, *cbv, splits, ws, out, stream);
}

int tq_decode_attention(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const float* q_rot,
                        const float* q_sketch, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                        float* out, float* scores, int split_tokens, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!out || !tq::aligned(out, 4)) return TQ_ERR_INVALID;
    // two launches: at the c4 shape (one round of workgroups) a separate combine costs less
    // than the in-launch merge's tail, whose record stores, arrival and record loads are three
    // memory round trips after the last workgroup of a stream (100.7 against 102.4 us a step)
    int st = tq_decode_partial(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, seq_lens, scores, split_tokens, ws,
                               ws_bytes, stream);
    if (st != TQ_OK) return st;
    return tq_decode_combine(L, cbv, split_tokens, ws, ws_bytes, out, stream);
}

int tq_decode_attention_hybrid(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const float* q_rot,
                               const float* q_sketch, const void* k_cache, const void* v_cache,
                               const int32_t* comp_lens, int ring_cap, const void* k_ring, const void* v_ring,
                               const int32_t* ring_lens, float* out, int split_tokens, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
    using namespace tq;
    if (!out || !k_ring || !v_ring || !ring_lens || !aligned(out, 4) || !aligned(ring_lens, 4) ||
        !aligned(k_ring, 16) || !aligned(v_ring, 16))
        return TQ_ERR_INVALID;
    if (ring_cap < 1 || ring_cap > kRingCapMax) return TQ_ERR_INVALID;
    int st = decode_partial(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, comp_lens, nullptr, split_tokens, ws,
                            ws_bytes, Launch{stream, nullptr, nullptr});
    if (st != TQ_OK) return st;
    int len = 0;
    const int splits = resolve_splits(L, split_tokens, &len);
    const RingView ring{q_rot, k_ring, v_ring, comp_lens, ring_lens, ring_cap};
    return combine(L, cbk, *cbv, splits, ws, out, stream, &ring);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode without a caller workspace, for callers that cannot allocate device memory
// (code under graph capture, tight serving loops): the split records live in a
// file-scope device array of fixed size, one copy per GPU the library runs on.  Its
// address is taken once per device (the array's name in host code is only a host-side
// stand-in) and kept per device.  All calls on one GPU share the array: calls that
// overlap on one GPU race.  The two-launch decode needs nothing in it to start at zero.

namespace tq {
namespace {

constexpr size_t kStaticScratchBytes = TQ_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once known

// The current device's copy of the scratch array (taken with that device current).
int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TQ_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return TQ_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TQ_OK;
}

}  // namespace
}  // namespace tq

extern "C" int tq_decode_attention_static(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv,
                                          const float* q_rot, const float* q_sketch, const void* k_cache,
                                          const void* v_cache, const int32_t* seq_lens, float* out,
                                          int split_tokens, hipStream_t stream) {
    using namespace tq;
    const size_t need = workspace_bytes(L, split_tokens);
    if (need == 0) return L && check_layout(L) != TQ_OK ? check_layout(L) : TQ_ERR_INVALID;
    if (need > kStaticScratchBytes) return TQ_ERR_WORKSPACE;  // before any HIP call
    void* ws = nullptr;
    const int st = scratch_of_current_device(&ws);
    if (st != TQ_OK) return st;
    return tq_decode_attention(L, cbk, cbv, q_rot, q_sketch, k_cache, v_cache, seq_lens, out, nullptr, split_tokens,
                               ws, kStaticScratchBytes, stream);
}
