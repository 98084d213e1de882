// Merge of the decode split records on gfx950, and the ring part of the
// hybrid read.  See decode_combine_kernel below.

#include <hip/hip_runtime.h>

#include <cmath>

#include "tq_device.h"

namespace tq {
namespace {

// ---------------------------------------------------------------------------
// Merge of the split records, and the ring part of hybrid attention.
//
// One workgroup per (b, query head) row merges the row's split records,
// normalizes and, for rotated value formats, rotates back once.  Each thread
// owns four coordinates of one split group and merges its records with a
// running maximum of its own, so every record load is issued before any
// maximum is known.
//
// With a capture ring (RMAX > 0) the same workgroup also attends over the
// ring's exact fp16 tokens ([P2] "write path": the newest tokens stay exact in
// a ring buffer until a batch is flushed into compressed blocks, and the
// hybrid mode reads both): exact scores against q = Pi_k^T q_rot in the log2
// units of the records, a softmax over the ring, and value sums in the
// unrotated basis, which join the merge after the rotation back (the rotation
// is linear).  The ring's rows are staged in LDS: key rows with their 16-byte
// pieces swizzled by the token (piece c of token t at c ^ (t & 15)), so that
// the one or two threads of a token read them free of bank conflicts; value
// rows in plain order.  When both do not fit (d = 256 with 256 ring tokens)
// the value rows are loaded after the scores, into the key buffer.
constexpr int kCombineThreads = 256;
static_assert(kRingCapMax <= kCombineThreads, "one or two threads per ring token");

struct CombineArgs {
    const float2* ml;
    const float* acc;
    float* out;
    int splits;  // records per row
    // capture ring, hybrid read only
    const float* q_rot;
    const uint16_t* k_ring;
    const uint16_t* v_ring;
    const int32_t* comp_lens;
    const int32_t* ring_lens;
    int hq;
    int hkv;
    int ring_cap;
};

template <int D, int RMAX>
struct RingStage {
    static constexpr int KPT = D / 8;                        // 16-byte pieces per row
    static constexpr int PPT = RMAX * KPT / kCombineThreads;  // pieces per thread
    static constexpr bool VLATE = 2 * RMAX * KPT * 16 > 128 * 1024;
    static constexpr int TPT = RMAX > 0 ? kCombineThreads / RMAX : 1;  // threads per ring token
    static_assert(RMAX == 0 || (RMAX * KPT) % kCombineThreads == 0, "whole pieces per thread");
    static_assert(RMAX == 0 || (TPT * RMAX == kCombineThreads && KPT % TPT == 0), "ring split over threads");
};

// 16-byte piece e of a ring's rows (key or value) in token order; tokens past n
// read the newest row (the oldest when the ring is empty), which keeps every
// load inside the ring.
template <int D>
__device__ __forceinline__ uint4 load_ring_piece(const uint16_t* ring, int ring_cap, size_t row0, int first, int nl,
                                                 int e) {
    const int t = min(e / (D / 8), nl);
    const int slot = (first + t) % ring_cap;
    return reinterpret_cast<const uint4*>(ring + (row0 + slot) * D)[e % (D / 8)];
}

template <int D, bool ROTATED, int RMAX>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(CombineArgs a, DevCodebook cbk,
                                                                        DevCodebook cbv) {
    constexpr int TPR = D / 4;                    // threads per record row
    constexpr int NGS = kCombineThreads / TPR;    // split groups
    constexpr int DPL = D / 64;
    constexpr int NW = kCombineThreads / 64;
    constexpr float kInvSqrtD = D == 256 ? 0.0625f : 0.08838834764831845f;
    using S = RingStage<D, RMAX>;
    constexpr int KPT = S::KPT, PPT = S::PPT, TPT = S::TPT;
    constexpr bool RING = RMAX > 0, VLATE = S::VLATE;
    constexpr int NTG = kCombineThreads / (D / 2);  // token groups of the ring's value sums
    constexpr int KR = RING ? RMAX : 1, KC = RING ? KPT : 1;
    __shared__ float4 part[NGS][TPR];
    __shared__ float part_m[NGS], part_l[NGS];
    __shared__ float fin_ml[2];
    __shared__ float o_sh[D];
    __shared__ float qs[RING ? D : 1];               // q = Pi_k^T q_rot times log2(e)/sqrt(d)
    __shared__ float pw[KR];                         // 2^(s - m) per ring token
    __shared__ float red_m[NW], red_l[NW];
    __shared__ float accp[RING ? NTG : 1][RING ? D : 1];  // ring value sums per token group
    __shared__ uint4 kst[KR][KC];                    // ring key rows, swizzled
    __shared__ uint4 vst_own[RING && !VLATE ? RMAX : 1][KC];
    uint4(*vst)[KC] = VLATE ? kst : vst_own;

    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    // ---- ring loads first: they are in flight while the records merge
    int n = 0, nl = 0, first = 0;
    size_t row0 = 0;
    float qv[DPL];
    uint4 kraw[RING ? PPT : 1], vraw[RING && !VLATE ? PPT : 1];
    if constexpr (RING) {
        const int b = row / a.hq, h = (row % a.hq) / (a.hq / a.hkv);
        n = a.ring_lens[b];
        n = n < 0 ? 0 : (n > a.ring_cap ? a.ring_cap : n);
        nl = max(n - 1, 0);
        first = max(a.comp_lens[b], 0);  // absolute position of the oldest ring token
        row0 = (static_cast<size_t>(b) * a.hkv + h) * a.ring_cap;
#pragma unroll
        for (int k = 0; k < DPL; ++k) qv[k] = a.q_rot[static_cast<size_t>(row) * D + DPL * lane + k];
#pragma unroll
        for (int i = 0; i < PPT; ++i)
            kraw[i] = load_ring_piece<D>(a.k_ring, a.ring_cap, row0, first, nl, i * kCombineThreads + tid);
        if constexpr (!VLATE) {
#pragma unroll
            for (int i = 0; i < PPT; ++i)
                vraw[i] = load_ring_piece<D>(a.v_ring, a.ring_cap, row0, first, nl, i * kCombineThreads + tid);
        }
    }

    // ---- split records: running maximum per thread, batches of SPT records whose
    // loads are all issued first (indexes past the last record reread it, weight 0)
    constexpr int SPT = 4;
    const int grp = tid / TPR, c = tid % TPR;
    const float2* mr = a.ml + static_cast<size_t>(row) * a.splits;
    const float4* ar = reinterpret_cast<const float4*>(a.acc) + static_cast<size_t>(row) * a.splits * TPR + c;
    float Mt = -INFINITY, Lt = 0.0f;
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int s0 = grp; s0 < a.splits; s0 += SPT * NGS) {
        float2 r[SPT];
        float4 v[SPT];
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int s = min(s0 + u * NGS, a.splits - 1);
            r[u] = mr[s];
            v[u] = ar[static_cast<size_t>(s) * TPR];
        }
        float mb = Mt;
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            if (s0 + u * NGS >= a.splits) r[u].x = -INFINITY;  // empty splits and the reread weigh nothing
            mb = fmaxf(mb, r[u].x);
        }
        // selects, not branches, keep the value loads ahead of the maxima
        const bool none = mb == -INFINITY;
        const float so = none ? 1.0f : exp2f(Mt - mb);  // 0 while nothing has been merged
        Lt *= so;
        o.x *= so; o.y *= so; o.z *= so; o.w *= so;
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const float f = r[u].x == -INFINITY ? 0.0f : exp2f(r[u].x - mb);
            Lt = fmaf(r[u].y, f, Lt);
            o.x = fmaf(v[u].x, f, o.x); o.y = fmaf(v[u].y, f, o.y);
            o.z = fmaf(v[u].z, f, o.z); o.w = fmaf(v[u].w, f, o.w);
        }
        Mt = mb;
    }
    part[grp][c] = o;
    if (c == 0) {
        part_m[grp] = Mt;
        part_l[grp] = Lt;
    }

    float Mr = -INFINITY, Lr = 0.0f;
    if constexpr (RING) {
        if (w == 0) {
            wht_wave<DPL>(qv, lane);
#pragma unroll
            for (int k = 0; k < DPL; ++k)
                qs[DPL * lane + k] = qv[k] * kInvSqrtD * rotation_sign(cbk, DPL * lane + k) * (kLog2e * kInvSqrtD);
        }
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int e = i * kCombineThreads + tid, t = e / KPT, cc = e % KPT;
            kst[t][cc ^ (t & 15)] = kraw[i];
        }
        if constexpr (!VLATE) {
#pragma unroll
            for (int i = 0; i < PPT; ++i) {
                const int e = i * kCombineThreads + tid;
                vst[e / KPT][e % KPT] = vraw[i];
            }
        }
    }
    __syncthreads();

    if constexpr (RING) {
        // exact scores: TPT adjacent lanes per token, each over KPT / TPT pieces
        const int t = tid / TPT, hf = tid % TPT;
        float sc = 0.0f;
#pragma unroll 4
        for (int i = 0; i < KPT / TPT; ++i) {
            const int cc = hf * (KPT / TPT) + i;
            const uint4 kp = kst[t][cc ^ (t & 15)];
            const uint32_t wd[4] = {kp.x, kp.y, kp.z, kp.w};
            const float4 q0 = *reinterpret_cast<const float4*>(&qs[8 * cc]);
            const float4 q1 = *reinterpret_cast<const float4*>(&qs[8 * cc + 4]);
            const float qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) sc = fmaf(qq[e], half_bits_to_float((wd[e >> 1] >> (16 * (e & 1))) & 0xFFFFu), sc);
        }
        if constexpr (TPT == 2) sc += __shfl_xor(sc, 1, 64);
        const bool live = t < n;
        const float mw = wave_max(live ? sc : -INFINITY);
        if (lane == 0) red_m[w] = mw;
        __syncthreads();
        Mr = red_m[0];
#pragma unroll
        for (int i = 1; i < NW; ++i) Mr = fmaxf(Mr, red_m[i]);
        const float p = live ? exp2f(sc - Mr) : 0.0f;
        if (hf == 0) pw[t] = p;
        const float lw = wave_sum(hf == 0 ? p : 0.0f);
        if (lane == 0) red_l[w] = lw;
        if constexpr (VLATE) {  // the key rows have been read: the value rows take their place
#pragma unroll
            for (int i = 0; i < PPT; ++i)
                kraw[i] = load_ring_piece<D>(a.v_ring, a.ring_cap, row0, first, nl, i * kCombineThreads + tid);
            __syncthreads();
#pragma unroll
            for (int i = 0; i < PPT; ++i) {
                const int e = i * kCombineThreads + tid;
                vst[e / KPT][e % KPT] = kraw[i];
            }
        }
        __syncthreads();
        Lr = 0.0f;
#pragma unroll
        for (int i = 0; i < NW; ++i) Lr += red_l[i];

        // value sums over the exact fp16 rows: coordinate pair jp, tokens tg, tg + NTG, ...
        const int jp = tid % (D / 2), tg = tid / (D / 2);
        const uint32_t* vs = reinterpret_cast<const uint32_t*>(&vst[0][0]);
        float2 av = make_float2(0.0f, 0.0f);
#pragma unroll 4
        for (int tt = tg; tt < n; tt += NTG) {
            const float pp = pw[tt];
            const uint32_t v2 = vs[tt * (D / 2) + jp];
            av.x = fmaf(pp, half_bits_to_float(v2 & 0xFFFFu), av.x);
            av.y = fmaf(pp, half_bits_to_float(v2 >> 16), av.y);
        }
        accp[tg][2 * jp] = av.x;
        accp[tg][2 * jp + 1] = av.y;
    }

    // ---- merge of the split groups (in the records' basis)
    if (tid < TPR) {
        float M = part_m[0];
#pragma unroll
        for (int g = 1; g < NGS; ++g) M = fmaxf(M, part_m[g]);
        float4 t = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float L = 0.0f;
        if (M != -INFINITY) {
#pragma unroll
            for (int g = 0; g < NGS; ++g) {
                const float f = exp2f(part_m[g] - M);
                const float4 u = part[g][tid];
                t.x = fmaf(u.x, f, t.x); t.y = fmaf(u.y, f, t.y);
                t.z = fmaf(u.z, f, t.z); t.w = fmaf(u.w, f, t.w);
                L = fmaf(part_l[g], f, L);
            }
        }
        o_sh[4 * tid] = t.x;
        o_sh[4 * tid + 1] = t.y;
        o_sh[4 * tid + 2] = t.z;
        o_sh[4 * tid + 3] = t.w;
        if (tid == 0) {
            fin_ml[0] = M;
            fin_ml[1] = L;
        }
    }
    __syncthreads();
    if (tid >= 64) return;
    float v[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) v[k] = o_sh[DPL * lane + k];
    if constexpr (ROTATED) {  // o <- Pi^T o = diag(s) H o / sqrt(d)
        wht_wave<DPL>(v, lane);
#pragma unroll
        for (int k = 0; k < DPL; ++k) v[k] *= kInvSqrtD * rotation_sign(cbv, DPL * lane + k);
    }
    const float Mc = fin_ml[0], Lc = fin_ml[1];
    float wc = 1.0f, wr = 0.0f, L = Lc;
    if constexpr (RING) {
        const float M = fmaxf(Mc, Mr);
        wc = Mc == -INFINITY ? 0.0f : exp2f(Mc - M);
        wr = Mr == -INFINITY ? 0.0f : exp2f(Mr - M);
        L = Lc * wc + Lr * wr;
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
        float x = v[k] * wc;
        if constexpr (RING) {
            float r = 0.0f;
#pragma unroll
            for (int g = 0; g < NTG; ++g) r += accp[g][DPL * lane + k];
            x = fmaf(r, wr, x);
        }
        a.out[static_cast<size_t>(row) * D + DPL * lane + k] = x * inv;
    }
}

template <int D, bool ROT>
void launch_combine(const CombineArgs& a, int rows, int rmax, const DevCodebook& ck, const DevCodebook& cv,
                    hipStream_t st) {
    const dim3 grid(rows), block(kCombineThreads);
    if (rmax == 0) hipLaunchKernelGGL((decode_combine_kernel<D, ROT, 0>), grid, block, 0, st, a, ck, cv);
    else if (rmax == 128) hipLaunchKernelGGL((decode_combine_kernel<D, ROT, 128>), grid, block, 0, st, a, ck, cv);
    else hipLaunchKernelGGL((decode_combine_kernel<D, ROT, 256>), grid, block, 0, st, a, ck, cv);
}

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, size_t n) {
    const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace

int clear_words(uint32_t* p, size_t n, hipStream_t stream) {
    if (n == 0) return TQ_OK;
    hipLaunchKernelGGL(clear_words_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, p, n);
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

int combine(const tq_layout* L, const tq_codebook* cbk, const tq_codebook& cbv, int splits, const void* ws, float* out,
            hipStream_t stream, const RingView* ring) {
    static_assert(kRingCapMax <= 256, "combine kernels are built for up to 256 ring tokens");
    const WsLayout wl = ws_layout(*L, splits);
    CombineArgs a{};
    a.ml = static_cast<const float2*>(ws);
    a.acc = reinterpret_cast<const float*>(static_cast<const char*>(ws) + wl.acc);
    a.out = out;
    a.splits = splits;
    a.hq = L->n_q_heads;
    a.hkv = L->n_kv_heads;
    int rmax = 0;
    if (ring) {
        a.q_rot = ring->q_rot;
        a.k_ring = static_cast<const uint16_t*>(ring->k_ring);
        a.v_ring = static_cast<const uint16_t*>(ring->v_ring);
        a.comp_lens = ring->comp_lens;
        a.ring_lens = ring->ring_lens;
        a.ring_cap = ring->ring_cap;
        rmax = ring->ring_cap <= 128 ? 128 : 256;
    }
    const int rows = L->batch * L->n_q_heads;
    const bool rot = !is_group_quant(L->v_format);
    const DevCodebook cv = to_dev(cbv), ck = cbk ? to_dev(*cbk) : cv;
    if (L->head_dim == 128) {
        if (rot) launch_combine<128, true>(a, rows, rmax, ck, cv, stream);
        else launch_combine<128, false>(a, rows, rmax, ck, cv, stream);
    } else {
        if (rot) launch_combine<256, true>(a, rows, rmax, ck, cv, stream);
        else launch_combine<256, false>(a, rows, rmax, ck, cv, stream);
    }
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

}  // namespace tq
