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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
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

// One wavefront per (b, query head): merge split records, normalize, rotate back.
template <int D, bool ROTATED>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float2* __restrict__ ml, const float* __restrict__ acc,
                                                           float* __restrict__ out, int splits, DevCodebook cbv) {
    constexpr int DPL = D / 64;
    const int row = blockIdx.x, lane = threadIdx.x;
    const float2* mr = ml + static_cast<size_t>(row) * splits;
    float M = -INFINITY;
    for (int s = lane; s < splits; s += 64) M = fmaxf(M, mr[s].x);
    M = wave_max(M);
    float o[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] = 0.0f;
    float L = 0.0f;
    if (M != -INFINITY) {
        const float* ar = acc + static_cast<size_t>(row) * splits * D;
        for (int s = 0; s < splits; ++s) {
            const float2 r = mr[s];
            if (r.x == -INFINITY) continue;
            const float f = exp2f(r.x - M);
            L = fmaf(r.y, f, L);
#pragma unroll
            for (int k = 0; k < DPL; ++k) o[k] = fmaf(ar[static_cast<size_t>(s) * D + lane * DPL + k], f, o[k]);
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] *= inv;
    if constexpr (ROTATED) {
        // o <- Pi^T o = diag(s) H o / sqrt(d); element j = DPL*lane + k
#pragma unroll
        for (int st = 1; st < DPL; st <<= 1)
#pragma unroll
            for (int k = 0; k < DPL; ++k)
                if ((k & st) == 0) {
                    const float x = o[k], y = o[k + st];
                    o[k] = x + y;
                    o[k + st] = x - y;
                }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const bool upper = (lane & m) != 0;
#pragma unroll
            for (int k = 0; k < DPL; ++k) {
                const float p = __shfl_xor(o[k], m, 64);
                o[k] = upper ? (p - o[k]) : (o[k] + p);
            }
        }
        constexpr float kInvSqrtD = D == 256 ? 0.0625f : 0.08838834764831845f;
#pragma unroll
        for (int k = 0; k < DPL; ++k) o[k] *= kInvSqrtD * rotation_sign(cbv, DPL * lane + k);
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) out[static_cast<size_t>(row) * D + DPL * lane + k] = o[k];
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

template <int KF, int VF, int D>
int dispatch_group(int G, const DecodeArgs& a, const tq_layout* L, const tq_codebook& cbk, const tq_codebook& cbv,
                   hipStream_t st) {
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
        if (rot) hipLaunchKernelGGL((decode_combine_kernel<128, true>), dim3(rows), dim3(64), 0, stream, ml, acc, out, splits, c);
        else hipLaunchKernelGGL((decode_combine_kernel<128, false>), dim3(rows), dim3(64), 0, stream, ml, acc, out, splits, c);
    } else {
        if (rot) hipLaunchKernelGGL((decode_combine_kernel<256, true>), dim3(rows), dim3(64), 0, stream, ml, acc, out, splits, c);
        else hipLaunchKernelGGL((decode_combine_kernel<256, false>), dim3(rows), dim3(64), 0, stream, ml, acc, out, splits, c);
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
