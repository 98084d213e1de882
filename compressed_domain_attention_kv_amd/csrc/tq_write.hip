// Write path of libtq on gfx950: quantize-and-append, quantize from given
// rotated coordinates, and the once-per-query rotation / QJL sketch.
//
// One vector is spread over LPV = d/8 lanes holding 8 consecutive
// coordinates each, so the fp16 row is read with one 16-byte load per lane
// (fully coalesced) and the Walsh-Hadamard transform runs 3 butterfly
// stages in registers and log2(LPV) stages across lanes.  Norms and group
// min/max are lane-group reductions.  Codes are packed in registers and
// stored as whole dwords / halfwords of the block.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "tq_device.h"
#include "tq_pq4.h"


namespace tq {
namespace {

constexpr int kWriteThreads = 256;
constexpr int kWriteThreadsC = kWriteThreads;

// kFp16Rows: fp16 rows x[nvec][d], destination row from dst_row (append);
// kRotated: fp32 rotated rows y with given norms, dense output (code test);
// kRing: fp16 rows gathered from the capture ring (flush).
enum class Src { kFp16Rows, kRotated, kRing };

struct WriteArgs {
    const uint16_t* x;        // fp16 rows [nvec][d] (Src::kFp16Rows)
    const float* y;           // fp32 rotated rows [nvec][d] (Src::kRotated)
    const uint16_t* norm16;   // fp16 norms [nvec] (Src::kRotated)
    const int32_t* dst_row;   // [nvec / hkv] rows, or null for dense output
    const float* S;           // d x d QJL matrix (TQ3K)
    uint8_t* out;
    int nvec;
    int hkv;
    int capacity;
    int batch;
    // kRing: vector (t, h) with t = b * count + i is token first[b] + i of the ring
    const int32_t* first;
    int ring_cap;
    int count;
    // floor(2^32 / d) (2^32 - 1 for d = 1) of the divisors hkv, capacity, count, ring_cap
    uint32_t hkv_m, cap_m, count_m, ring_m;
};

// The reciprocals of a write's divisors (host side, once per call).
uint32_t div_magic(int d) {
    return d <= 1 ? 0xFFFFFFFFu : static_cast<uint32_t>((uint64_t{1} << 32) / static_cast<uint64_t>(d));
}
void set_divisors(WriteArgs& a) {
    a.hkv_m = div_magic(a.hkv);
    a.cap_m = div_magic(a.capacity);
    a.count_m = div_magic(a.count);
    a.ring_m = div_magic(a.ring_cap);
}

// q = n / d and r = n % d for 0 <= n < 2^31 and d >= 1, given m = floor(2^32 / d) (2^32 - 1
// for d = 1): mulhi(n, m) is floor(n / d) or one less (n m / 2^32 lies within n / 2^32 < 1 below
// n / d), and one remainder test settles which.
__device__ __forceinline__ void divmod(int n, int d, uint32_t m, int& q, int& r) {
    uint32_t qq = __umulhi(static_cast<uint32_t>(n), m);
    uint32_t rr = static_cast<uint32_t>(n) - qq * static_cast<uint32_t>(d);
    if (rr >= static_cast<uint32_t>(d)) {
        ++qq;
        rr -= static_cast<uint32_t>(d);
    }
    q = static_cast<int>(qq);
    r = static_cast<int>(rr);
}

// Index of the first fp32 boundary not below y, i.e. #{k : bounds[k] < y}.
template <int NLEV>
__device__ __forceinline__ uint32_t code_of(float y, const DevCodebook& cb) {
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < NLEV - 1; ++k) c += (y > cb.bounds[k]) ? 1u : 0u;
    return c;
}

// Sketch rows of the vectors a workgroup holds in LDS: thread t owns row
// i = t % d of S and the vectors h, h + NH, ... with h = t / d (NH = 256 / d row
// groups); acc[k] = sum_j S[i][j] xs[h + NH k][j], summed over j in order four
// at a time.  Every thread streams its own row of S, so the loads are independent
// and the vectors are LDS broadcasts.
template <int D, int NV>
__device__ __forceinline__ void sketch_rows(const float* __restrict__ S, const float* xs, int tid, float (&acc)[NV]) {
    constexpr int NH = kWriteThreadsC / D;
    const int i = tid % D, h = tid / D;
    const float4* srow = reinterpret_cast<const float4*>(S + static_cast<size_t>(i) * D);
#pragma unroll
    for (int k = 0; k < NV; ++k) acc[k] = 0.0f;
#pragma unroll 8
    for (int j = 0; j < D / 4; ++j) {
        const float4 s4 = srow[j];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const float4 x4 = reinterpret_cast<const float4*>(xs + (h + NH * k) * D)[j];
            acc[k] += s4.x * x4.x + s4.y * x4.y + s4.z * x4.z + s4.w * x4.w;
        }
    }
}

template <int FMT>
struct FormatTraits;
template <>
struct FormatTraits<TQ_FMT_PQ4> { static constexpr int kLevels = 16; };
template <>
struct FormatTraits<TQ_FMT_PQ3> { static constexpr int kLevels = 8; };
template <>
struct FormatTraits<TQ_FMT_TQ3K> { static constexpr int kLevels = 4; };
template <>
struct FormatTraits<TQ_FMT_GQ2V> { static constexpr int kLevels = 4; };
template <>
struct FormatTraits<TQ_FMT_GQ4V> { static constexpr int kLevels = 16; };

template <int FMT, int D>
constexpr int vec_bytes_c() {
    return FMT == TQ_FMT_PQ4 ? 68 * (D / 128)
         : FMT == TQ_FMT_PQ3 ? 14 * (D / 32)
         : FMT == TQ_FMT_TQ3K ? 4 + D / 4 + D / 8
         : FMT == TQ_FMT_GQ2V ? 12 * (D / kGroup)
                              : 20 * (D / kGroup);
}

// Vectors per lane group handled by one workgroup pass: every one of them has its
// source row requested before the first is encoded, so a wavefront keeps U rows in
// flight instead of paying one memory latency per row.
constexpr int kWriteUnroll = 8;

// Where vector `vec` of a write goes (byte offset of its block) and which source
// row it reads; inactive vectors (past nvec, bad destination) compute on row 0
// and store nothing.
template <int FMT, int D, Src SRC>
struct VecTarget {
    bool active;
    size_t off;
    size_t src_row;
};

template <int FMT, int D, Src SRC>
__device__ __forceinline__ VecTarget<FMT, D, SRC> vec_target(const WriteArgs& a, int vec) {
    constexpr int VB = vec_bytes_c<FMT, D>();
    VecTarget<FMT, D, SRC> t{vec < a.nvec, 0, 0};
    if constexpr (SRC == Src::kRing) {
        int tk, h, bb, i;
        divmod(t.active ? vec : 0, a.hkv, a.hkv_m, tk, h);
        divmod(tk, a.count, a.count_m, bb, i);
        const int f = a.first[bb];
        const int pos = f + i;
        if (!t.active || f < 0 || pos >= a.capacity) t.active = false;
        else t.off = ((static_cast<size_t>(bb) * a.hkv + h) * a.capacity + pos) * VB;
        int wrap, slot;
        divmod(t.active ? pos : 0, a.ring_cap, a.ring_m, wrap, slot);
        t.src_row = t.active ? (static_cast<size_t>(bb) * a.hkv + h) * a.ring_cap + slot : 0;
    } else {
        t.src_row = t.active ? static_cast<size_t>(vec) : 0;
        if (t.active) {
            if (a.dst_row) {
                int tk, h;
                divmod(vec, a.hkv, a.hkv_m, tk, h);
                const int r = a.dst_row[tk];
                if (r < 0 || r >= a.batch * a.capacity) {
                    t.active = false;
                } else {
                    int b, pos;
                    divmod(r, a.capacity, a.cap_m, b, pos);
                    t.off = ((static_cast<size_t>(b) * a.hkv + h) * a.capacity + pos) * VB;
                }
            } else {
                t.off = static_cast<size_t>(vec) * VB;
            }
        }
    }
    return t;
}

// The source row of vector `vec`, without its destination: any row of the write for a vector
// that stores nothing (fp16 rows: the vector itself, so the row loads need not wait for the
// destination rows; ring: as vec_target finds it).
template <int FMT, int D, Src SRC>
__device__ __forceinline__ size_t src_row_of(const WriteArgs& a, int vec) {
    if constexpr (SRC == Src::kRing) return vec_target<FMT, D, SRC>(a, vec).src_row;
    else return vec < a.nvec ? static_cast<size_t>(vec) : 0;
}

// The 8 coordinates 8l .. 8l+7 of one source row, as loaded (not yet converted).
struct RowPiece {
    uint4 x;        // fp16 rows
    float4 y0, y1;  // fp32 rotated rows
    uint32_t n16;   // their stored norm
};

template <int D, Src SRC>
__device__ __forceinline__ RowPiece load_piece(const WriteArgs& a, size_t row, int l) {
    RowPiece p{};
    if constexpr (SRC != Src::kRotated) {
        p.x = *reinterpret_cast<const uint4*>(a.x + row * D + 8 * l);
    } else {
        const float4* src = reinterpret_cast<const float4*>(a.y + row * D + 8 * l);
        p.y0 = src[0];
        p.y1 = src[1];
        p.n16 = a.norm16[row];
    }
    return p;
}

// Rotation signs of coordinates 8l .. 8l+7 (one byte of the sign words).
__device__ __forceinline__ uint32_t sign_byte(const DevCodebook& cb, int l) {
    return (cb.sign_bits[l >> 2] >> (8 * (l & 3))) & 0xFFu;
}

// Encode one vector from its loaded piece and store its block.
template <int FMT, int D, Src SRC>
__device__ __forceinline__ void encode_vec(const WriteArgs& a, const DevCodebook& cb, const VecTarget<FMT, D, SRC>& tg,
                                           const RowPiece& in, uint32_t sgn, int l, int slot, float* r_sh,
                                           uint64_t* qjl_sh) {
    constexpr int LPV = D / 8;
    const bool active = tg.active;
    float v[8];
    uint32_t n16 = 0;
    if constexpr (SRC != Src::kRotated) {
        const uint32_t w[4] = {in.x.x, in.x.y, in.x.z, in.x.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = half_bits_to_float((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    } else {
        v[0] = in.y0.x; v[1] = in.y0.y; v[2] = in.y0.z; v[3] = in.y0.w;
        v[4] = in.y1.x; v[5] = in.y1.y; v[6] = in.y1.z; v[7] = in.y1.w;
        n16 = in.n16;
    }

    uint8_t* dst = a.out + tg.off;
    if constexpr (FMT == TQ_FMT_GQ2V || FMT == TQ_FMT_GQ4V) {
        // asymmetric 2- or 4-bit group quantization, groups of 32 channels = 4 lanes:
        // zero = min, scale = (max - min) / (levels - 1), codes by rounding to the grid
        constexpr int QMAX = FormatTraits<FMT>::kLevels - 1, QB = FMT == TQ_FMT_GQ2V ? 2 : 4;
        constexpr int GB = 4 + kGroup * QB / 8;  // bytes per group
        float mn = v[0], mx = v[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) { mn = fminf(mn, v[e]); mx = fmaxf(mx, v[e]); }
#pragma unroll
        for (int m = 1; m < 4; m <<= 1) {
            mn = fminf(mn, __shfl_xor(mn, m, LPV));
            mx = fmaxf(mx, __shfl_xor(mx, m, LPV));
        }
        const uint32_t z16 = float_to_half_bits(mn);  // exact: mn is an fp16 value
        const uint32_t s16 = float_to_half_bits(__fdiv_rn(mx - mn, static_cast<float>(QMAX)));
        const float z = half_bits_to_float(z16), s = half_bits_to_float(s16);
        // no branches: with inv = 0 (scale 0, or NaN) every code is 0 (fmaxf(NaN, 0) = 0), as it
        // is by definition for a zero scale
        const float inv_s = __fdiv_rn(1.0f, s);
        const float inv = s > 0.0f ? inv_s : 0.0f;
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // clamp to [0, QMAX] in one median (a NaN product gives 0, as the min-max pair did)
            const float t = __builtin_amdgcn_fmed3f(rintf((v[e] - z) * inv), 0.0f, static_cast<float>(QMAX));
            packed |= static_cast<uint32_t>(t) << (QB * e);
        }
        if (active) {
            const int grp = l >> 2, lg = l & 3;
            uint8_t* g = dst + GB * grp;
            if (lg == 0) *reinterpret_cast<uint32_t*>(g) = s16 | (z16 << 16);
            if constexpr (QB == 2) *reinterpret_cast<uint16_t*>(g + 4 + 2 * lg) = static_cast<uint16_t>(packed);
            else *reinterpret_cast<uint32_t*>(g + 4 + 4 * lg) = packed;
        }
    } else {
        constexpr float kInvSqrtD = D == 256 ? 0.0625f : 0.08838834764831845f;
        if constexpr (SRC != Src::kRotated) {
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
            ss = group_sum<LPV>(ss);
            const float n = sqrtf(ss);
            n16 = float_to_half_bits(fminf(n, kFp16Max));
            const float inv = n > 0.0f ? __fdiv_rn(1.0f, n) : 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = v[e] * inv * (((sgn >> e) & 1u) ? -1.0f : 1.0f);
            wht8<LPV>(v, l);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= kInvSqrtD;
        }
        constexpr int NLEV = FormatTraits<FMT>::kLevels;
        uint32_t code[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) code[e] = code_of<NLEV>(v[e], cb);

        if constexpr (FMT == TQ_FMT_PQ4) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) word |= code[e] << (4 * e);
            if (active) {
                const int blk = l >> 4, lb = l & 15;
                uint8_t* bp = dst + 68 * blk;
                if (lb == 0) *reinterpret_cast<uint32_t*>(bp) = n16;
                *reinterpret_cast<uint32_t*>(bp + 4 + 4 * lb) = word;
            }
        } else if constexpr (FMT == TQ_FMT_PQ3) {
            uint32_t low = 0, high = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                low |= (code[e] & 3u) << (2 * e);
                high |= ((code[e] >> 2) & 1u) << e;
            }
            if (active) {
                const int blk = l >> 2, lb = l & 3;
                uint8_t* bp = dst + 14 * blk;
                if (lb == 0) *reinterpret_cast<uint16_t*>(bp) = static_cast<uint16_t>(n16);
                *reinterpret_cast<uint16_t*>(bp + 2 + 2 * lb) = static_cast<uint16_t>(low);
                bp[10 + lb] = static_cast<uint8_t>(high);
            }
        } else {  // TQ3K: 2-bit MSE codes plus the QJL sketch of the residual
            uint32_t low = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) low |= code[e] << (2 * e);
            // residual in the rotated basis, rotated back: r = Pi^T (y - c)
            float r[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) r[e] = v[e] - cb.centroids[code[e]];
            wht8<LPV>(r, l);
            float g2 = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                r[e] = r[e] * kInvSqrtD * (((sgn >> e) & 1u) ? -1.0f : 1.0f);
                g2 += r[e] * r[e];
            }
            g2 = group_sum<LPV>(g2);
            const uint32_t g16 = float_to_half_bits(fminf(sqrtf(g2), kFp16Max));
            float* rs = r_sh + slot * D;
#pragma unroll
            for (int e = 0; e < 8; ++e) rs[8 * l + e] = r[e];
            __syncthreads();
            // b_i = [(S r)_i >= 0]: the sketch rows per thread, the bits of 64 rows of one
            // vector gathered by a ballot into LDS, where lane l finds its byte (rows 8l..8l+7)
            constexpr int VPB = kWriteThreads / LPV, NH = kWriteThreads / D, NV = VPB / NH;
            float acc[NV];
            sketch_rows<D, NV>(a.S, r_sh, threadIdx.x, acc);
            const int lane = threadIdx.x & 63, row0 = (threadIdx.x % D) & ~63, h = threadIdx.x / D;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const uint64_t m = __builtin_amdgcn_ballot_w64(acc[k] >= 0.0f);
                if (lane == 0) qjl_sh[(h + NH * k) * (D / 64) + row0 / 64] = m;
            }
            __syncthreads();
            const uint32_t bits = reinterpret_cast<const uint8_t*>(qjl_sh + slot * (D / 64))[l];
            __syncthreads();  // residuals and bits are read before the next vector writes them
            if (active) {
                if (l == 0) *reinterpret_cast<uint32_t*>(dst) = n16 | (g16 << 16);
                *reinterpret_cast<uint16_t*>(dst + 4 + 2 * l) = static_cast<uint16_t>(low);
                dst[4 + D / 4 + l] = static_cast<uint8_t>(bits);
            }
        }
    }
}


// The vectors of workgroup `block` of one quantize grid: kWriteUnroll passes of
// kWriteThreads / (d / 8) vectors.
template <int FMT, int D, Src SRC>
__device__ __forceinline__ void quantize_rows(const WriteArgs& a, const DevCodebook& cb, int block) {
    constexpr int LPV = D / 8;                  // lanes per vector
    constexpr int VPB = kWriteThreads / LPV;    // vectors per pass
    constexpr int U = kWriteUnroll;
    __shared__ float r_sh[FMT == TQ_FMT_TQ3K ? VPB * D : 1];
    __shared__ uint64_t qjl_sh[FMT == TQ_FMT_TQ3K ? VPB * D / 64 : 1];  // sketch bits per vector
    const int tid = threadIdx.x;
    const int l = tid % LPV;
    const int slot = tid / LPV;
    const uint32_t sgn = sign_byte(cb, l);
    VecTarget<FMT, D, SRC> tg[U];
#pragma unroll
    for (int u = 0; u < U; ++u) tg[u] = vec_target<FMT, D, SRC>(a, (block * U + u) * VPB + slot);
    RowPiece in[U];
#pragma unroll
    for (int u = 0; u < U; ++u) in[u] = load_piece<D, SRC>(a, src_row_of<FMT, D, SRC>(a, (block * U + u) * VPB + slot), l);
#pragma unroll
    for (int u = 0; u < U; ++u) encode_vec<FMT, D, SRC>(a, cb, tg[u], in[u], sgn, l, slot, r_sh, qjl_sh);
}

// ---------------------------------------------------------------------------
// PQ4 from fp16 rows (append, bulk prefill, ring flush): lane l of a vector holds
// the 16 consecutive coordinates j = 16 l + e, so four Walsh-Hadamard stages run
// in registers and the rest (lane bits 1, 2, 4, 8 inside a row of 16 lanes) are
// DPP lane moves folded into the adds, as is the norm's sum: the vector never
// passes through LDS.  The rotation signs flip the fp16 sign bits before the
// conversion, and one scale 1 / (n sqrt(d)) follows the norm.  Each lane packs
// its 8 code bytes and stores them with one 8-byte store.
// 16 coordinates per lane (8 lanes per vector at d = 128, 16 at d = 256) and four
// passes per workgroup whose loads are issued first.  The kernel is bound by VALU
// issue (about 35 instructions per coordinate: norm, 7-8 butterfly stages, the
// four-level code search, packing); lanes per vector and passes per workgroup
// from 4 to 16 and 1 to 8 measured within 5% of each other.
template <int D>
constexpr int pq4_lanes() { return D / 16; }
// passes per workgroup: four for bulk writes; one when the launch is small (an append of
// a token per stream), so each wavefront's chain of VALU work is a quarter as long
template <int D>
constexpr int pq4_unroll() { return 4; }
constexpr int kPq4SmallVectors = 8192;  // at most this many vectors: one pass per workgroup
template <int D, Src SRC, int U>
__global__ __launch_bounds__(kWriteThreads) void quantize_pq4_kernel(WriteArgs ak, WriteArgs av, DevCodebook cbk,
                                                                     DevCodebook cbv, int kblocks) {
    static_assert(SRC != Src::kRotated, "fp16 sources");
    constexpr int LANES = pq4_lanes<D>();
    constexpr int CPL = D / LANES;                // coordinates per lane
    constexpr int NPC = CPL / 8;                  // 16-byte pieces of fp16 input per lane
    constexpr int VPP = kWriteThreads / LANES;    // vectors per pass
    // copies chosen by a uniform condition (a reference chosen at run time would put the
    // kernel arguments in scratch memory)
    const bool is_k = static_cast<int>(blockIdx.x) < kblocks;
    const WriteArgs a = is_k ? ak : av;
    const DevCodebook cb = is_k ? cbk : cbv;
    const int block = is_k ? blockIdx.x : blockIdx.x - kblocks;
    const int tid = threadIdx.x, l = tid % LANES, slot = tid / LANES;

    uint32_t smask[CPL / 2];
    // rotation signs of this lane's coordinates CPL l .. CPL l + CPL - 1 (selected, not indexed:
    // an indexed array of the words would be placed in LDS or scratch)
    uint32_t sw = cb.sign_bits[0];
#pragma unroll
    for (int i = 1; i < D / 32; ++i)
        if ((CPL * l) >> 5 == i) sw = cb.sign_bits[i];
    pq4_sign_masks<CPL>(CPL == 32 ? sw : (sw >> ((CPL * l) & 31)) & 0xFFFFu, smask);
    __shared__ float4 sb4[4];  // boundaries b0 .. b14 (and +inf)
    if (tid < 16)  // indexed in the arguments, not in a copy
        reinterpret_cast<float*>(sb4)[tid] = tid < 15 ? (is_k ? cbk.bounds[tid] : cbv.bounds[tid]) : INFINITY;
    const float b3 = cb.bounds[3], b7 = cb.bounds[7], b11 = cb.bounds[11];
    __syncthreads();

    VecTarget<TQ_FMT_PQ4, D, SRC> tg[U];
#pragma unroll
    for (int u = 0; u < U; ++u) tg[u] = vec_target<TQ_FMT_PQ4, D, SRC>(a, (block * U + u) * VPP + slot);
    uint4 raw[U][NPC];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int c = 0; c < NPC; ++c)
            raw[u][c] = *reinterpret_cast<const uint4*>(
                a.x + src_row_of<TQ_FMT_PQ4, D, SRC>(a, (block * U + u) * VPP + slot) * D + CPL * l + 8 * c);

#pragma unroll
    for (int u = 0; u < U; ++u) {
        uint32_t n16, words[CPL / 8];
        pq4_encode<D, LANES>(raw[u], smask, b3, b7, b11, sb4, l, n16, words);
        if (tg[u].active) pq4_store<D, LANES>(a.out + tg[u].off, l, n16, words);
    }
}

// ---------------------------------------------------------------------------
// PQ4 at d = 256 on the matrix cores.  The Sylvester transform of order 256 is
// H[c'][c] = (-1)^popcount(c' & c), so splitting the 8 index bits into any two groups of four
// makes it the Kronecker square of the order-16 one: with coordinate c = 64 g + 4 a + e
// (a in 0..15, g and e in 0..3) read as M[a][4g + e] = s_c x_c, the rotated row is
// Y = H16 M H16 / (16 n) with y_(64 g' + 4 a' + e') = Y[a'][4g' + e'] ([P1] section 1: norm,
// normalize, rotate, nearest centroid); this split lets lane l read bytes 8l .. 8l+7 of the row.  M H16 is one fp16 product
// (the inputs and the +-1 entries are exact in fp16, the sums fp32); its fp32 result, scaled
// by 1 / (16 n), is already laid out as the second operand of H16 (M H16) and enters it as an
// fp16 part plus the fp16 rounding of the remainder (two more products), so nothing moves
// between lanes.  The codes come from a
// 64-cell table: cell(y) = clamp(trunc(A y + B)) is monotone in y and each cell holds at
// most one boundary (the host checks this in the same fp32 arithmetic), so
// #{k : b_k < y} = #{k : cell(b_k) < cell(y)} + (y > the boundary of cell(y)).

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
    const auto a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[0], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[1], a[1], false, false);
    out[0] = b[0];
    out[1] = b[1];
    out[2] = c[0];
    out[3] = c[1];
}

constexpr int kLutCells = 64, kLutCopies = 32;  // one copy per LDS bank pair
constexpr int kD256Rows = 64;                   // rows per chunk: one row target per lane
constexpr int kD256Chunks = 1;                  // chunks per wavefront
constexpr int kD256Unroll = 4;                  // rows in flight per wavefront

__device__ __forceinline__ uint32_t lut_cell(float y, float A, float B) {
    return static_cast<uint32_t>(__builtin_amdgcn_fmed3f(fmaf(y, A, B), 0.0f, static_cast<float>(kLutCells - 1)));
}

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

template <Src SRC>
__global__ __launch_bounds__(kWriteThreads) __attribute__((amdgpu_waves_per_eu(4))) void quantize_pq4_d256_kernel(
    WriteArgs ak, WriteArgs av, DevCodebook cbk, DevCodebook cbv, int kblocks, int nblocks) {
    static_assert(SRC != Src::kRotated, "fp16 sources");
    constexpr int D = 256, U = kD256Unroll, NW = kWriteThreads / 64;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: row targets stay scalar
    const int li = lane & 15, lg = lane >> 4;  // row of M (a) / column of the products (j); lane group

    __shared__ uint2 lut[kLutCells * kLutCopies];  // (boundary bits, #{k : cell(b_k) < cell}) of (cell, copy)
    __shared__ uint2 cells[kLutCells];
    __shared__ uint8_t codes[NW][U][D];            // codes of the rows in flight, by coordinate

    // H16[r][c] = (-1)^popcount(r & c): the second operand of M H16 (lane (j, g): H16[4g + i][j])
    // is, H16 being symmetric, also the first operand of H16 (M H16) (lane (i, g): H16[i][4g + t])
    half4_t hb;
#pragma unroll
    for (int t = 0; t < 4; ++t) hb[t] = static_cast<_Float16>((__builtin_popcount((4 * lg + t) & li) & 1) ? -1.0f : 1.0f);

    // Workgroups stay resident and take blocks of NW x 64 rows in turn: the key blocks first, then
    // the value blocks, so a workgroup builds each table at most once.
    int table = -1;  // 0: the keys' table is in LDS, 1: the values'
    float A = 0.0f, B = 0.0f;
    uint32_t sm0 = 0, sm1 = 0;
    for (int blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
    const bool is_k = blk < kblocks;
    // copies chosen by a uniform condition (a reference chosen at run time would put the kernel
    // arguments in scratch memory)
    const WriteArgs a = is_k ? ak : av;
    const int block = is_k ? blk : blk - kblocks;
    if (table != (is_k ? 0 : 1)) {
        table = is_k ? 0 : 1;
        const DevCodebook cb = is_k ? cbk : cbv;
        A = static_cast<float>(kLutCells - 2) / (cb.bounds[14] - cb.bounds[0]);
        B = fmaf(-cb.bounds[0], A, 1.0f);
        __syncthreads();  // the previous table's last lookups are done
        if (tid < kLutCells) {
            uint32_t k0 = 0;
            float bs = INFINITY;
#pragma unroll
            for (int k = 0; k < 15; ++k) {
                const uint32_t ck = lut_cell(cb.bounds[k], A, B);
                k0 += ck < static_cast<uint32_t>(tid) ? 1u : 0u;
                bs = ck == static_cast<uint32_t>(tid) ? cb.bounds[k] : bs;
            }
            cells[tid] = make_uint2(__float_as_uint(bs), k0);
        }
        // this lane's rotation signs (coordinates 64 lg + 4 li .. + 3; the word selected, not
        // indexed, so the arguments stay out of scratch) as XOR masks of its two fp16 pairs
        uint32_t sw = cb.sign_bits[0];
#pragma unroll
        for (int i = 1; i < 8; ++i)
            if (2 * lg + (li >> 3) == i) sw = cb.sign_bits[i];
        const uint32_t s4 = (sw >> (4 * (li & 7))) & 0xFu;
        sm0 = ((s4 & 1u) << 15) | (((s4 >> 1) & 1u) << 31);
        sm1 = (((s4 >> 2) & 1u) << 15) | (((s4 >> 3) & 1u) << 31);
        __syncthreads();
        for (int i = tid; i < kLutCells * kLutCopies; i += kWriteThreads) lut[i] = cells[i / kLutCopies];
        __syncthreads();
    }

    // the wavefront's chunks of 64 rows: lane i finds the target of row i of a chunk once,
    // rows read it by lane
    static_assert(kD256Rows == 64, "one row target per lane");
    const uint32_t copy = lane & (kLutCopies - 1);
    for (int chunk = 0; chunk < kD256Chunks; ++chunk) {
    const int vbase = ((block * NW + wv) * kD256Chunks + chunk) * kD256Rows;
    const VecTarget<TQ_FMT_PQ4, D, SRC> mine = vec_target<TQ_FMT_PQ4, D, SRC>(a, vbase + lane);
    const uint64_t active_rows = __builtin_amdgcn_ballot_w64(mine.active);
    const size_t src_mine = src_row_of<TQ_FMT_PQ4, D, SRC>(a, vbase + lane);
    const uint32_t src_lo = static_cast<uint32_t>(src_mine), src_hi = static_cast<uint32_t>(src_mine >> 32);
    const uint32_t off_lo = static_cast<uint32_t>(mine.off), off_hi = static_cast<uint32_t>(mine.off >> 32);
    auto src_of = [&](int r) __attribute__((always_inline)) {
        return static_cast<size_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(src_lo, r))) |
               static_cast<size_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(src_hi, r))) << 32;
    };
    auto load_rows = [&](uint2 (&dst)[U], int first) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            dst[u] = *reinterpret_cast<const uint2*>(a.x + src_of(first + u) * D + 4 * lane);
    };
    uint2 raw[U], nxt[U];
    load_rows(nxt, 0);
    for (int it = 0; it < kD256Rows; it += U) {
        // each stage runs over the U rows in flight, so the products of one row overlap the
        // work on the others; the next rows' loads are in flight meanwhile
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = nxt[u];
        if (it + U < kD256Rows) load_rows(nxt, it + U);
        uint32_t x01[U], x23[U];
        float ss[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            x01[u] = raw[u].x ^ sm0;
            x23[u] = raw[u].y ^ sm1;
            const half2_t h01 = __builtin_bit_cast(half2_t, x01[u]), h23 = __builtin_bit_cast(half2_t, x23[u]);
            ss[u] = __builtin_amdgcn_fdot2(h23, h23, __builtin_amdgcn_fdot2(h01, h01, 0.0f, false), false);
        }
        f32x4_t p[U], y[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            p[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, make_uint2(x01[u], x23[u])), hb,
                                                         f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        // the four norms at once: after a transpose across the lane groups, lane group g holds
        // the partial sums of row g from all four groups; their sum over the group's 16 lanes is
        // row g's squared norm, whose root and reciprocal every lane group takes for its row
        static_assert(U % 4 == 0, "one row per lane group");
        constexpr int NG = U / 4;
        uint32_t scl[U], n16g[NG];
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            uint32_t part[4] = {__float_as_uint(ss[4 * q]), __float_as_uint(ss[4 * q + 1]),
                                __float_as_uint(ss[4 * q + 2]), __float_as_uint(ss[4 * q + 3])};
            group_transpose(part);
            float sq = (__uint_as_float(part[0]) + __uint_as_float(part[1])) +
                       (__uint_as_float(part[2]) + __uint_as_float(part[3]));
            sq += lane_xor<1>(sq);
            sq += lane_xor<2>(sq);
            sq += lane_xor<4>(sq);
            sq += lane_xor<8>(sq);
            // the hardware root and reciprocal (within an ulp of the rounded results): the norm's
            // fp16 rounding can move only within 1e-7 of an fp16 midpoint, y by under 1e-7 relative
            const float n = __builtin_amdgcn_sqrtf(sq);
            n16g[q] = float_to_half_bits(fminf(n, kFp16Max));
            const float scale_g = (n > 0.0f ? __builtin_amdgcn_rcpf(n) : 0.0f) * 0.0625f;  // 1 / (n sqrt(256))
            uint32_t b4[4];
            group_broadcast(__float_as_uint(scale_g), b4);
#pragma unroll
            for (int i = 0; i < 4; ++i) scl[4 * q + i] = b4[i];
        }
        // H16 P1 / (16 n) as two fp16 products: P1 / (16 n) (at most 1/4 in size) split into an
        // fp16 part and the fp16 rounding of its remainder, 22 significant bits together
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float sc = __uint_as_float(scl[u]);
            const float v0 = p[u][0] * sc, v1 = p[u][1] * sc, v2 = p[u][2] * sc, v3 = p[u][3] * sc;
            const half2_t h01 = __builtin_convertvector((float2_t{v0, v1}), half2_t);
            const half2_t h23 = __builtin_convertvector((float2_t{v2, v3}), half2_t);
            const half2_t l01 = __builtin_convertvector(
                (float2_t{v0 - static_cast<float>(h01[0]), v1 - static_cast<float>(h01[1])}), half2_t);
            const half2_t l23 = __builtin_convertvector(
                (float2_t{v2 - static_cast<float>(h23[0]), v3 - static_cast<float>(h23[1])}), half2_t);
            const half4_t hi{h01[0], h01[1], h23[0], h23[1]}, lo{l01[0], l01[1], l23[0], l23[1]};
            y[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(hb, hi, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            y[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(hb, lo, y[u], 0, 0, 0);
        }
        // y[u][r] = Y[4 lg + r][li] of row u: rotated coordinate 64 (li / 4) + 16 lg + 4 r + li % 4
        const int cbase = 64 * (li >> 2) + 16 * lg + (li & 3);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint2 e = lut[lut_cell(y[u][r], A, B) * kLutCopies + copy];
                codes[wv][u][cbase + 4 * r] = static_cast<uint8_t>(e.y + (y[u][r] > __uint_as_float(e.x) ? 1u : 0u));
            }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // lanes 0..31 pack coordinates 8 lane .. 8 lane + 7 into a code word of the lane's block;
        // lanes 32, 33 write the [fp16 norm][0] headers of blocks 0 and 1
        const bool packer = lane < 32;
        const uint32_t dst_off = packer ? 68 * (lane >> 4) + 4 + 4 * (lane & 15) : 68 * (lane - 32);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint2 c8 = *reinterpret_cast<const uint2*>(&codes[wv][u][8 * (lane & 31)]);
            const uint32_t t0 = c8.x | (c8.x >> 4), t1 = c8.y | (c8.y >> 4);  // bytes 0, 2: two codes each
            const uint32_t word =
                packer ? __builtin_amdgcn_perm(t1, t0, 0x06040200u) : __builtin_amdgcn_readlane(n16g[u / 4], 16 * (u % 4));
            const size_t off = static_cast<size_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(off_lo, it + u))) |
                               static_cast<size_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(off_hi, it + u))) << 32;
            if (((active_rows >> (it + u)) & 1u) && lane < 34) *reinterpret_cast<uint32_t*>(a.out + off + dst_off) = word;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    }
    }
}

template <int FMT, int D, Src SRC>
__global__ __launch_bounds__(kWriteThreads) void quantize_kernel(WriteArgs a, DevCodebook cb) {
    quantize_rows<FMT, D, SRC>(a, cb, blockIdx.x);
}

// Keys and values of one append in one launch when they share a format: the
// first kblocks workgroups take the keys, the rest the values.
template <int FMT, int D, Src SRC>
__global__ __launch_bounds__(kWriteThreads) void quantize_kv_kernel(WriteArgs ak, WriteArgs av, DevCodebook cbk,
                                                                    DevCodebook cbv, int kblocks) {
    if (static_cast<int>(blockIdx.x) < kblocks)
        quantize_rows<FMT, D, SRC>(ak, cbk, blockIdx.x);
    else
        quantize_rows<FMT, D, SRC>(av, cbv, blockIdx.x - kblocks);
}

// Capture ring append: row (b, h) of the new token goes to ring slot pos[b] % ring_cap.
// One thread moves 16 bytes; a sequence with pos < 0 is skipped.
__global__ __launch_bounds__(kWriteThreads) void ring_append_kernel(const uint4* __restrict__ k_new,
                                                                    const uint4* __restrict__ v_new,
                                                                    const int32_t* __restrict__ pos, uint4* k_ring,
                                                                    uint4* v_ring, int batch, int hkv, int chunks,
                                                                    int ring_cap) {
    const int i = blockIdx.x * kWriteThreads + threadIdx.x;  // over 2 tensors x batch x hkv x chunks
    const int per_tensor = batch * hkv * chunks;
    if (i >= 2 * per_tensor) return;
    const int tensor = i / per_tensor, j = i % per_tensor;
    const int row = j / chunks, c = j % chunks;
    const int b = row / hkv, h = row % hkv;
    const int p = pos[b];
    if (p < 0) return;
    const size_t dst = ((static_cast<size_t>(b) * hkv + h) * ring_cap + p % ring_cap) * chunks + c;
    if (tensor == 0) k_ring[dst] = k_new[j];
    else v_ring[dst] = v_new[j];
}

// q_rot = Pi q = H (s * q) / sqrt(d); for TQ3K keys also q_sketch = S q.  With the
// sketch the grid has D / RPW workgroups per group of VPB queries along y: workgroup
// y writes rows y RPW .. y RPW + RPW - 1 of the sketch, one (row, query) dot
// product per thread (the queries of a row are consecutive threads, so they read
// the same row of S), and workgroup y = 0 also writes q_rot.
template <int D>
constexpr int sketch_rows_per_wg() { return kWriteThreads / (kWriteThreads / (D / 8)); }

template <int D, bool SKETCH>
__global__ __launch_bounds__(kWriteThreads) void rotate_query_kernel(const float* __restrict__ q, float* __restrict__ q_rot,
                                                                  float* __restrict__ q_sk, const float* __restrict__ S,
                                                                  int nvec, DevCodebook cb) {
    constexpr int LPV = D / 8;
    constexpr int VPB = kWriteThreads / LPV;
    constexpr float kInvSqrtD = D == 256 ? 0.0625f : 0.08838834764831845f;
    constexpr int QS = D + 4;  // padded rows: the queries of one row read distinct banks
    __shared__ float q_sh[SKETCH ? VPB * QS : 1];
    const int tid = threadIdx.x, l = tid % LPV, slot = tid / LPV;
    const int vec = blockIdx.x * VPB + slot;
    const bool active = vec < nvec;
    const int vsrc = active ? vec : 0;
    const float4* src = reinterpret_cast<const float4*>(q + static_cast<size_t>(vsrc) * D + 8 * l);
    const float4 p0 = src[0], p1 = src[1];
    float v[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    if constexpr (SKETCH) {
#pragma unroll
        for (int e = 0; e < 8; ++e) q_sh[slot * QS + 8 * l + e] = v[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= rotation_sign(cb, 8 * l + e);
    wht8<LPV>(v, l);
    if (active && blockIdx.y == 0) {
        float4* o = reinterpret_cast<float4*>(q_rot + static_cast<size_t>(vec) * D + 8 * l);
        o[0] = make_float4(v[0] * kInvSqrtD, v[1] * kInvSqrtD, v[2] * kInvSqrtD, v[3] * kInvSqrtD);
        o[1] = make_float4(v[4] * kInvSqrtD, v[5] * kInvSqrtD, v[6] * kInvSqrtD, v[7] * kInvSqrtD);
    }
    if constexpr (SKETCH) {
        __syncthreads();
        constexpr int RPW = sketch_rows_per_wg<D>();
        const int i = blockIdx.y * RPW + tid / VPB, k = tid % VPB;
        const float4* srow = reinterpret_cast<const float4*>(S + static_cast<size_t>(i) * D);
        const float4* xq = reinterpret_cast<const float4*>(q_sh + k * QS);
        float acc = 0.0f;
#pragma unroll 8
        for (int j = 0; j < D / 4; ++j) {
            const float4 s4 = srow[j], x4 = xq[j];
            acc += s4.x * x4.x + s4.y * x4.y + s4.z * x4.z + s4.w * x4.w;
        }
        const int vk = blockIdx.x * VPB + k;
        if (vk < nvec) q_sk[static_cast<size_t>(vk) * D + i] = acc;
    }
}

// ---------------------------------------------------------------------------
// TQ3K keys at d = 128 on the matrix cores ([P2] write path: 2-bit MSE codes of the rotated
// unit vector, then the sign bits of S r for the residual r rotated back, with its norm
// gamma).  A workgroup takes batches of 64 vectors, each wavefront two vectors at a time:
//   1. Rotation.  H_128 = H_8 (x) H_16 for coordinate c = 16 a + b.  The 16 x 16 fp16 matrix
//      M of two vectors (row 8 v + a, column b; the rotation signs applied to the fp16 sign
//      bits) is loaded with 8 bytes per lane; one product gives P = M H_16 (exact inputs,
//      fp32 sums), which is scaled by 1 / (n sqrt(d)) per vector and split into an fp16 part
//      and the fp16 rounding of its remainder (22 significant bits); a second product, with
//      P in the operand position of its transpose, gives Y^T = P^T diag(H_8, H_8), so lane
//      (j, g) ends up with coordinates 16 (j & 7) + 4 g .. + 3 of vector j >> 3.
//   2. Codes by the three boundaries, the residual r' = y - c in the rotated basis and
//      gamma = |r'| (the rotation is orthogonal: |r| = |r'|); the codes, the [n16 | gamma16]
//      header and r' (scaled by 2^10, a power of two: the signs do not change, and its small
//      entries stay normal fp16 numbers, as an fp16 part and remainder) go to LDS.
//   3. Sketch.  S r = S Pi^T r' = S' r' with S' = S diag(s) H / sqrt(d), formed once per
//      workgroup from S and held in registers as fp16 parts and remainders (wavefront w: rows
//      32 w .. 32 w + 31), so r is never rotated back; S' R' for the batch on the fp16 matrix
//      cores, hi*hi + hi*lo + lo*hi (a sign flips only where |(S r)_i| is within about 1e-6 of
//      |S_i| |r|); each row's sign goes to LDS as a byte already shifted to its bit of the
//      output byte.
//   4. Four threads per vector OR 8 of those bytes into each sketch byte and write the block.
constexpr int kTq3kBatch = 64;   // vectors per batch
constexpr int kTq3kRow = 136;    // halves per residual row in LDS (16 B of padding: distinct banks)
constexpr int kTq3kSgnRow = 132; // bytes per sign row in LDS

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

// x as a materialized fp32 value.  An fp16 part and remainder of a product must both be
// taken from its fp32 rounding: left to itself the compiler forms the part by a fused
// multiply-convert of the exact product (one rounding) and the remainder against the other,
// and the two disagree by an fp16 ulp whenever the two roundings differ.
__device__ __forceinline__ float rounded(float x) {
    asm("" : "+v"(x));
    return x;
}

// Sum over the 32 lanes of one vector of a pair: lanes 8 v .. 8 v + 7 of every row of 16
// lanes (v = 0, 1); the eight inside a row by DPP moves, the four rows by two lane swaps.
__device__ __forceinline__ float pair_vector_sum(float x) {
    x += lane_xor<1>(x);
    x += lane_xor<2>(x);
    x += lane_xor<4>(x);
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(h[0]) + __uint_as_float(h[1]);  // rows 0 + 2 and 1 + 3, in both halves
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <Src SRC>
__global__ __launch_bounds__(kWriteThreads) void quantize_tq3k_mfma_kernel(WriteArgs a, DevCodebook cb, int nbatches) {
    static_assert(SRC != Src::kRotated, "fp16 sources");
    constexpr int D = 128, NB = kTq3kBatch, NW = kWriteThreads / 64, PPW = NB / NW / 2;  // vector pairs per wavefront
    constexpr int U = 4;                                                                  // pairs in flight
    constexpr float kInvSqrtD = 0.08838834764831845f, kRScale = 1024.0f;
    // the rotated coordinates are formed as 2^8 y (exact power-of-two scaling), so that the
    // fp16 remainders of the second product stay normal numbers; boundaries and centroids
    // are scaled alike
    constexpr float kYs = 256.0f;
    __shared__ __align__(16) _Float16 rhi[NB][kTq3kRow];
    __shared__ __align__(16) _Float16 rlo[NB][kTq3kRow];
    __shared__ __align__(16) uint8_t sgn_sh[NB][kTq3kSgnRow];
    __shared__ __align__(16) uint32_t blk_sh[NB][9];  // per vector: n16 | gamma16 << 16, then the 8 code dwords
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;  // MFMA row / column, k group

    // ---- S' = S diag(s) H / sqrt(d): rows 32 wv + 16 rt + li, columns 32 c + 8 lg + e, as
    // fp16 part and remainder.  The column's bits e (0-2) and c (5-6) are in registers, lg
    // (3-4) across the lane groups.
    half8_t shi[2][4], slo[2][4];
    {
        uint32_t sb[4];  // bit e: the sign of column 32 c + 8 lg + e
#pragma unroll
        for (int c = 0; c < 4; ++c) sb[c] = cb.sign_bits[c] >> (8 * lg);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float x[4][8];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float4* src = reinterpret_cast<const float4*>(a.S + (32 * wv + 16 * rt + li) * D + 32 * c + 8 * lg);
                const float4 p0 = src[0], p1 = src[1];
                const float f[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) x[c][e] = ((sb[c] >> e) & 1u) ? -f[e] : f[e];
            }
#pragma unroll
            for (int st = 1; st < 8; st <<= 1)
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if ((e & st) == 0) {
                            const float u = x[c][e], v = x[c][e + st];
                            x[c][e] = u + v;
                            x[c][e + st] = u - v;
                        }
#pragma unroll
            for (int st = 1; st < 4; st <<= 1)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if ((c & st) == 0)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float u = x[c][e], v = x[c + st][e];
                            x[c][e] = u + v;
                            x[c + st][e] = u - v;
                        }
#pragma unroll
            for (int m = 16; m < 64; m <<= 1)
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float p = __shfl_xor(x[c][e], m);
                        x[c][e] = (lane & m) ? p - x[c][e] : x[c][e] + p;
                    }
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float f = rounded(x[c][e] * kInvSqrtD);
                    shi[rt][c][e] = static_cast<_Float16>(f);
                    slo[rt][c][e] = static_cast<_Float16>(f - static_cast<float>(shi[rt][c][e]));
                }
        }
    }

    // H16 (second operand of M H16: lane (j, g) holds H16[4g + t][j]) and diag(H8, H8)
    // (second operand of P^T diag(H8, H8), rows 4g + t, column j)
    half4_t h16, d8;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = 4 * lg + t;
        h16[t] = static_cast<_Float16>((__builtin_popcount(r & li) & 1) ? -1.0f : 1.0f);
        d8[t] = static_cast<_Float16>((r >> 3) != (li >> 3) ? 0.0f : (__builtin_popcount(r & li & 7) & 1) ? -1.0f : 1.0f);
    }
    // this lane's rotation signs (coordinates 16 (li & 7) + 4 lg .. + 3: word (li & 7) / 2, the
    // word selected, not indexed, so the arguments stay out of scratch) as XOR masks of its
    // two fp16 pairs
    const int aa = li & 7;
    uint32_t sw = cb.sign_bits[0];
#pragma unroll
    for (int i = 1; i < 4; ++i)
        if ((aa >> 1) == i) sw = cb.sign_bits[i];
    const uint32_t s4 = (sw >> (16 * (aa & 1) + 4 * lg)) & 0xFu;
    const uint32_t sm0 = ((s4 & 1u) << 15) | (((s4 >> 1) & 1u) << 31);
    const uint32_t sm1 = (((s4 >> 2) & 1u) << 15) | (((s4 >> 3) & 1u) << 31);
    const float m0 = cb.bounds[0] * kYs, m1 = cb.bounds[1] * kYs, m2 = cb.bounds[2] * kYs;
    const float c0 = cb.centroids[0] * kYs, c1 = cb.centroids[1] * kYs, c2 = cb.centroids[2] * kYs,
                c3 = cb.centroids[3] * kYs;

    // the source rows of a batch, as this lane holds them: the wavefront's vectors 16 wv ..
    // 16 wv + 15, pair pp = vectors 2 pp (lanes with li < 8) and 2 pp + 1.  A batch's rows are
    // requested during the previous batch.
    uint2 raw[PPW];
    auto load_rows = [&](int batch) __attribute__((always_inline)) {
#pragma unroll
        for (int pp = 0; pp < PPW; ++pp) {
            const size_t row = src_row_of<TQ_FMT_TQ3K, D, SRC>(a, batch * NB + 16 * wv + 2 * pp + (li >> 3));
            raw[pp] = *reinterpret_cast<const uint2*>(a.x + row * D + 16 * aa + 4 * lg);
        }
    };
    if (static_cast<int>(blockIdx.x) < nbatches) load_rows(blockIdx.x);

    for (int batch = blockIdx.x; batch < nbatches; batch += gridDim.x) {
        // where thread t's vector t / 4 goes (its destination row is read now, used at the end)
        const VecTarget<TQ_FMT_TQ3K, D, SRC> t4 = vec_target<TQ_FMT_TQ3K, D, SRC>(a, batch * NB + (tid >> 2));
        // ---- 1, 2. rotation, codes and residuals of the batch's vectors
#pragma unroll
        for (int q0 = 0; q0 < PPW; q0 += U) {
            f32x4_t y[U];
            uint32_t n16v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t x01 = raw[q0 + u].x ^ sm0, x23 = raw[q0 + u].y ^ sm1;
                const half2_t h01 = __builtin_bit_cast(half2_t, x01), h23 = __builtin_bit_cast(half2_t, x23);
                const float ss =
                    pair_vector_sum(__builtin_amdgcn_fdot2(h23, h23, __builtin_amdgcn_fdot2(h01, h01, 0.0f, false), false));
                // the hardware root and reciprocal (within an ulp of the rounded results: the
                // norm's fp16 rounding moves only within 1e-7 of an fp16 midpoint, y by under
                // 1e-7 relative)
                const float n = __builtin_amdgcn_sqrtf(ss);
                n16v[u] = float_to_half_bits(fminf(n, kFp16Max));  // of vector li >> 3
                const float sc = (n > 0.0f ? __builtin_amdgcn_rcpf(n) : 0.0f) * (kInvSqrtD * kYs);
                // rows 4 lg + r of M H16 belong to vector lg >> 1
                const float sc0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(sc), 0));
                const float sc1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(sc), 8));
                const float scl = lg < 2 ? sc0 : sc1;
                const f32x4_t pr = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, make_uint2(x01, x23)),
                                                                         h16, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                half4_t ph, pl;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = rounded(pr[r] * scl);
                    ph[r] = static_cast<_Float16>(v);
                    pl[r] = static_cast<_Float16>(v - static_cast<float>(ph[r]));
                }
                y[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, d8, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                y[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, d8, y[u], 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                // y[u][r]: 2^8 times coordinate 16 aa + 4 lg + r of vector li >> 3
                uint32_t byte = 0;
                float g2 = 0.0f;
                half4_t rh, rl;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = y[u][r];
                    const bool b0 = v > m0, b1 = v > m1, b2 = v > m2;  // code = #{k : m_k < y}
                    byte |= (static_cast<uint32_t>(b0) + static_cast<uint32_t>(b1) + static_cast<uint32_t>(b2)) << (2 * r);
                    const float res = v - (b1 ? (b2 ? c3 : c2) : (b0 ? c1 : c0));
                    g2 = fmaf(res, res, g2);
                    const float xs = res * (kRScale / kYs);
                    rh[r] = static_cast<_Float16>(xs);
                    rl[r] = static_cast<_Float16>(xs - static_cast<float>(rh[r]));
                }
                const uint32_t g16 =
                    float_to_half_bits(fminf(__builtin_amdgcn_sqrtf(pair_vector_sum(g2)) * (1.0f / kYs), kFp16Max));
                const int slot = 16 * wv + 2 * (q0 + u) + (li >> 3);  // the vector's place in the batch
                reinterpret_cast<uint8_t*>(blk_sh[slot])[4 + 4 * aa + lg] = static_cast<uint8_t>(byte);
                *reinterpret_cast<half4_t*>(&rhi[slot][16 * aa + 4 * lg]) = rh;
                *reinterpret_cast<half4_t*>(&rlo[slot][16 * aa + 4 * lg]) = rl;
                if (aa == 0 && lg == 0) blk_sh[slot][0] = n16v[u] | (g16 << 16);
            }
        }
        if (batch + static_cast<int>(gridDim.x) < nbatches) load_rows(batch + gridDim.x);
        __syncthreads();

        // ---- 3. signs of S' R': wavefront wv, rows 32 wv + 16 rt + 4 lg + i, vectors 16 ct + li
#pragma unroll
        for (int ct = 0; ct < NB / 16; ++ct) {
            f32x4_t acc[2] = {f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const half8_t bh = *reinterpret_cast<const half8_t*>(&rhi[16 * ct + li][32 * c + 8 * lg]);
                const half8_t bl = *reinterpret_cast<const half8_t*>(&rlo[16 * ct + li][32 * c + 8 * lg]);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(shi[rt][c], bh, acc[rt], 0, 0, 0);
                    acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(shi[rt][c], bl, acc[rt], 0, 0, 0);
                    acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(slo[rt][c], bh, acc[rt], 0, 0, 0);
                }
            }
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                uint32_t word = 0;  // byte i: row 4 lg + i of the tile, its bit of the sketch byte set when >= 0
#pragma unroll
                for (int i = 0; i < 4; ++i) word |= (acc[rt][i] >= 0.0f ? 1u : 0u) << (((4 * lg + i) & 7) + 8 * i);
                *reinterpret_cast<uint32_t*>(&sgn_sh[16 * ct + li][32 * wv + 16 * rt + 4 * lg]) = word;
            }
        }
        __syncthreads();

        // ---- 4. thread t, vector t / 4: sketch bytes 4 (t % 4) .. + 3 (rows 32 (t % 4) ..), code
        // dwords 2 (t % 4) and 2 (t % 4) + 1, and the header
        {
            const int v = tid >> 2, q = tid & 3;
            const uint32_t* sp = reinterpret_cast<const uint32_t*>(&sgn_sh[v][32 * q]);
            uint32_t out = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t x = sp[2 * j] | sp[2 * j + 1];
                x |= x >> 16;
                x |= x >> 8;
                out |= (x & 0xFFu) << (8 * j);
            }
            if (t4.active) {
                uint32_t* dst = reinterpret_cast<uint32_t*>(a.out + t4.off);  // blocks are 4-byte aligned
                dst[1 + D / 16 + q] = out;
                dst[1 + 2 * q] = blk_sh[v][1 + 2 * q];
                dst[2 + 2 * q] = blk_sh[v][2 + 2 * q];
                if (q == 0) dst[0] = blk_sh[v][0];
            }
        }
        __syncthreads();  // the batch's LDS is read before the next batch writes it
    }
}

// Workgroups of kWriteThreads threads of `kernel` that the current device holds at once
// (resident on every CU), found once per device and kernel.
template <typename K>
int resident_workgroups(K kernel) {
    struct Entry {
        const void* fn;
        int dev, count;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1 << 20;
    const void* fn = reinterpret_cast<const void*>(kernel);
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& e : cache)
        if (e.fn == fn && e.dev == dev) return e.count;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kWriteThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu < 1 || cus < 1)
        return 1 << 20;  // unknown: one workgroup per block
    cache.push_back({fn, dev, per_cu * cus});
    return per_cu * cus;
}

// Whether the 64-cell code table of quantize_pq4_d256_kernel serves a codebook: finite
// increasing boundaries b_0 .. b_14 whose cells, in the kernel's own fp32 arithmetic
// (A = 62 / (b_14 - b_0), B = fma(-b_0, A, 1), cell = clamp(trunc(fma(b, A, B)), 0, 63)),
// all differ, so no cell holds two boundaries.
bool pq4_lut_serves(const tq_codebook& cb) {
    for (int k = 0; k < 15; ++k)
        if (!std::isfinite(cb.bounds[k])) return false;
    if (!(cb.bounds[14] > cb.bounds[0])) return false;
    const float A = static_cast<float>(kLutCells - 2) / (cb.bounds[14] - cb.bounds[0]);
    const float B = std::fmaf(-cb.bounds[0], A, 1.0f);
    long prev = -1;
    for (int k = 0; k < 15; ++k) {
        const float t = std::fmin(std::fmax(std::fmaf(cb.bounds[k], A, B), 0.0f), static_cast<float>(kLutCells - 1));
        const long c = static_cast<long>(t);
        if (c <= prev) return false;
        prev = c;
    }
    return true;
}

// PQ4 from fp16 rows: keys (ak) and, when av.nvec > 0, values in one launch
template <int D, Src SRC>
int launch_pq4(const WriteArgs& ak, const WriteArgs& av, const tq_codebook& cbk, const tq_codebook& cbv,
               hipStream_t st) {
    constexpr int VPP = kWriteThreads / pq4_lanes<D>();  // vectors per pass
    if (ak.nvec + av.nvec == 0) return TQ_OK;
    if constexpr (D == 256) {
        if (pq4_lut_serves(cbk) && (av.nvec == 0 || pq4_lut_serves(cbv))) {
            constexpr int VPG = kWriteThreads / 64 * kD256Rows * kD256Chunks;  // vectors per block
            const int kblocks = (ak.nvec + VPG - 1) / VPG, vblocks = (av.nvec + VPG - 1) / VPG;
            const int grid = std::min(kblocks + vblocks, resident_workgroups(quantize_pq4_d256_kernel<SRC>));
            hipLaunchKernelGGL((quantize_pq4_d256_kernel<SRC>), dim3(grid), dim3(kWriteThreads), 0, st, ak, av,
                               to_dev(cbk), to_dev(cbv), kblocks, kblocks + vblocks);
            return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
        }
    }
    if (static_cast<long>(ak.nvec) + av.nvec <= kPq4SmallVectors) {
        const int kblocks = (ak.nvec + VPP - 1) / VPP, vblocks = (av.nvec + VPP - 1) / VPP;
        hipLaunchKernelGGL((quantize_pq4_kernel<D, SRC, 1>), dim3(kblocks + vblocks), dim3(kWriteThreads), 0, st, ak,
                           av, to_dev(cbk), to_dev(cbv), kblocks);
    } else {
        constexpr int VPG = VPP * pq4_unroll<D>();  // vectors per workgroup
        const int kblocks = (ak.nvec + VPG - 1) / VPG, vblocks = (av.nvec + VPG - 1) / VPG;
        hipLaunchKernelGGL((quantize_pq4_kernel<D, SRC, pq4_unroll<D>()>), dim3(kblocks + vblocks),
                           dim3(kWriteThreads), 0, st, ak, av, to_dev(cbk), to_dev(cbv), kblocks);
    }
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

template <int FMT, int D, Src SRC>
int launch_quantize(const WriteArgs& a, const tq_codebook& cb, hipStream_t st) {
    if constexpr (FMT == TQ_FMT_PQ4 && SRC != Src::kRotated) {
        WriteArgs none = a;
        none.nvec = 0;
        return launch_pq4<D, SRC>(a, none, cb, cb, st);
    }
    if constexpr (FMT == TQ_FMT_TQ3K && D == 128 && SRC != Src::kRotated) {
        const int nbatches = (a.nvec + kTq3kBatch - 1) / kTq3kBatch;
        if (nbatches == 0) return TQ_OK;
        const int grid = std::min(nbatches, resident_workgroups(quantize_tq3k_mfma_kernel<SRC>));
        hipLaunchKernelGGL((quantize_tq3k_mfma_kernel<SRC>), dim3(grid), dim3(kWriteThreads), 0, st, a, to_dev(cb),
                           nbatches);
        return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
    }
    constexpr int VPG = kWriteThreads / (D / 8) * kWriteUnroll;  // vectors per workgroup
    const int grid = (a.nvec + VPG - 1) / VPG;
    hipLaunchKernelGGL((quantize_kernel<FMT, D, SRC>), dim3(grid), dim3(kWriteThreads), 0, st, a, to_dev(cb));
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

template <int FMT, int D, Src SRC>
int launch_quantize_kv(const WriteArgs& ak, const WriteArgs& av, const tq_codebook& cbk, const tq_codebook& cbv,
                       hipStream_t st) {
    constexpr int VPG = kWriteThreads / (D / 8) * kWriteUnroll;  // vectors per workgroup
    const int kblocks = (ak.nvec + VPG - 1) / VPG;
    hipLaunchKernelGGL((quantize_kv_kernel<FMT, D, SRC>), dim3(2 * kblocks), dim3(kWriteThreads), 0, st, ak, av,
                       to_dev(cbk), to_dev(cbv), kblocks);
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

// Keys and values of one write: one launch when they share a format (PQ4, PQ3), else two.
template <Src SRC>
int quantize_pair(const tq_layout* L, const WriteArgs& ak, const WriteArgs& av, const tq_codebook& cbk,
                  const tq_codebook& cbv, hipStream_t stream);

template <Src SRC>
int dispatch_quantize(int fmt, int d, const WriteArgs& a, const tq_codebook& cb, hipStream_t st) {
#define TQ_Q(F)                                                                        \
    case F:                                                                            \
        return d == 128 ? launch_quantize<F, 128, SRC>(a, cb, st) : launch_quantize<F, 256, SRC>(a, cb, st);
    switch (fmt) {
        TQ_Q(TQ_FMT_PQ4)
        TQ_Q(TQ_FMT_PQ3)
        TQ_Q(TQ_FMT_TQ3K)
        default: break;
    }
    if constexpr (SRC != Src::kRotated) {
        if (fmt == TQ_FMT_GQ2V)
            return d == 128 ? launch_quantize<TQ_FMT_GQ2V, 128, SRC>(a, cb, st)
                            : launch_quantize<TQ_FMT_GQ2V, 256, SRC>(a, cb, st);
        if (fmt == TQ_FMT_GQ4V)
            return d == 128 ? launch_quantize<TQ_FMT_GQ4V, 128, SRC>(a, cb, st)
                            : launch_quantize<TQ_FMT_GQ4V, 256, SRC>(a, cb, st);
    }
#undef TQ_Q
    return TQ_ERR_UNSUPPORTED;
}

template <Src SRC>
int quantize_pair(const tq_layout* L, const WriteArgs& ak, const WriteArgs& av, const tq_codebook& cbk,
                  const tq_codebook& cbv, hipStream_t stream) {
    if (L->k_format == L->v_format && (L->k_format == TQ_FMT_PQ4 || L->k_format == TQ_FMT_PQ3)) {
        const bool d128 = L->head_dim == 128;
        if (L->k_format == TQ_FMT_PQ4) {
            if constexpr (SRC != Src::kRotated)
                return d128 ? launch_pq4<128, SRC>(ak, av, cbk, cbv, stream) : launch_pq4<256, SRC>(ak, av, cbk, cbv, stream);
            return d128 ? launch_quantize_kv<TQ_FMT_PQ4, 128, SRC>(ak, av, cbk, cbv, stream)
                        : launch_quantize_kv<TQ_FMT_PQ4, 256, SRC>(ak, av, cbk, cbv, stream);
        }
        return d128 ? launch_quantize_kv<TQ_FMT_PQ3, 128, SRC>(ak, av, cbk, cbv, stream)
                    : launch_quantize_kv<TQ_FMT_PQ3, 256, SRC>(ak, av, cbk, cbv, stream);
    }
    const int st = dispatch_quantize<SRC>(L->k_format, L->head_dim, ak, cbk, stream);
    if (st != TQ_OK) return st;
    return dispatch_quantize<SRC>(L->v_format, L->head_dim, av, cbv, stream);
}

}  // namespace
}  // namespace tq

extern "C" {

int tq_quantize_append(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const float* S_dev,
                       const uint16_t* k_new, const uint16_t* v_new, const int32_t* dst_row, int T, void* k_cache,
                       void* v_cache, hipStream_t stream) {
    using namespace tq;
    int st = check_layout(L);
    if (st != TQ_OK) return st;
    if (T < 0) return TQ_ERR_INVALID;
    if ((st = check_codebook(cbk, L->k_format, L->head_dim)) != TQ_OK) return st;
    if ((st = check_codebook(cbv, L->v_format, L->head_dim)) != TQ_OK) return st;
    if (T == 0) return TQ_OK;
    if (static_cast<double>(T) * L->n_kv_heads > 2147483647.0) return TQ_ERR_RANGE;
    if (!k_new || !v_new || !dst_row || !k_cache || !v_cache) return TQ_ERR_INVALID;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(dst_row, 4))
        return TQ_ERR_INVALID;
    if (L->k_format == TQ_FMT_TQ3K && (!S_dev || !aligned(S_dev, 16))) return TQ_ERR_INVALID;
    WriteArgs a{};
    a.dst_row = dst_row;
    a.S = S_dev;
    a.nvec = T * L->n_kv_heads;
    a.hkv = L->n_kv_heads;
    a.capacity = L->capacity;
    a.batch = L->batch;
    set_divisors(a);
    WriteArgs av = a;
    a.x = k_new;
    a.out = static_cast<uint8_t*>(k_cache);
    av.x = v_new;
    av.out = static_cast<uint8_t*>(v_cache);
    return quantize_pair<Src::kFp16Rows>(L, a, av, *cbk, *cbv, stream);
}

size_t tq_ring_bytes(const tq_layout* L, int ring_cap) {
    using namespace tq;
    if (check_layout(L) != TQ_OK || ring_cap < 1 || ring_cap > kRingCapMax) return 0;
    return static_cast<size_t>(L->batch) * L->n_kv_heads * ring_cap * L->head_dim * sizeof(uint16_t);
}

int tq_ring_append(const tq_layout* L, int ring_cap, const uint16_t* k_new, const uint16_t* v_new, const int32_t* pos,
                   void* k_ring, void* v_ring, hipStream_t stream) {
    using namespace tq;
    int st = check_layout(L);
    if (st != TQ_OK) return st;
    if (ring_cap < 1 || ring_cap > kRingCapMax) return TQ_ERR_INVALID;
    if (!k_new || !v_new || !pos || !k_ring || !v_ring) return TQ_ERR_INVALID;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_ring, 16) || !aligned(v_ring, 16) || !aligned(pos, 4))
        return TQ_ERR_INVALID;
    const int chunks = L->head_dim / 8;  // 16-byte pieces of one fp16 row
    const int total = 2 * L->batch * L->n_kv_heads * chunks;
    hipLaunchKernelGGL(ring_append_kernel, dim3((total + kWriteThreads - 1) / kWriteThreads), dim3(kWriteThreads), 0,
                       stream, static_cast<const uint4*>(static_cast<const void*>(k_new)),
                       static_cast<const uint4*>(static_cast<const void*>(v_new)), pos, static_cast<uint4*>(k_ring),
                       static_cast<uint4*>(v_ring), L->batch, L->n_kv_heads, chunks, ring_cap);
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

int tq_ring_flush(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const float* S_dev, int ring_cap,
                  const void* k_ring, const void* v_ring, const int32_t* first, int count, void* k_cache,
                  void* v_cache, hipStream_t stream) {
    using namespace tq;
    int st = check_layout(L);
    if (st != TQ_OK) return st;
    if ((st = check_codebook(cbk, L->k_format, L->head_dim)) != TQ_OK) return st;
    if ((st = check_codebook(cbv, L->v_format, L->head_dim)) != TQ_OK) return st;
    if (ring_cap < 1 || ring_cap > kRingCapMax || count < 0 || count > ring_cap) return TQ_ERR_INVALID;
    if (count == 0) return TQ_OK;
    if (!k_ring || !v_ring || !first || !k_cache || !v_cache) return TQ_ERR_INVALID;
    if (!aligned(k_ring, 16) || !aligned(v_ring, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(first, 4))
        return TQ_ERR_INVALID;
    if (L->k_format == TQ_FMT_TQ3K && (!S_dev || !aligned(S_dev, 16))) return TQ_ERR_INVALID;
    WriteArgs a{};
    a.S = S_dev;
    a.nvec = L->batch * count * L->n_kv_heads;
    a.hkv = L->n_kv_heads;
    a.capacity = L->capacity;
    a.batch = L->batch;
    a.first = first;
    a.ring_cap = ring_cap;
    a.count = count;
    set_divisors(a);
    WriteArgs av = a;
    a.x = static_cast<const uint16_t*>(k_ring);
    a.out = static_cast<uint8_t*>(k_cache);
    av.x = static_cast<const uint16_t*>(v_ring);
    av.out = static_cast<uint8_t*>(v_cache);
    return quantize_pair<Src::kRing>(L, a, av, *cbk, *cbv, stream);
}

int tq_quantize_rotated(int format, const tq_codebook* cb, const float* S_dev, const float* y, const uint16_t* norm16,
                        int n, void* blocks, hipStream_t stream) {
    using namespace tq;
    if (!cb) return TQ_ERR_INVALID;
    const int d = cb->head_dim;
    if (d != 128 && d != 256) return TQ_ERR_UNSUPPORTED;
    if (format != TQ_FMT_PQ4 && format != TQ_FMT_PQ3 && format != TQ_FMT_TQ3K) return TQ_ERR_UNSUPPORTED;
    int st = check_codebook(cb, format, d);
    if (st != TQ_OK) return st;
    if (n < 0) return TQ_ERR_INVALID;
    if (n == 0) return TQ_OK;
    if (!y || !norm16 || !blocks || !aligned(y, 16) || !aligned(blocks, 16) || !aligned(norm16, 2))
        return TQ_ERR_INVALID;
    if (format == TQ_FMT_TQ3K && (!S_dev || !aligned(S_dev, 16))) return TQ_ERR_INVALID;
    WriteArgs a{};
    a.y = y;
    a.norm16 = norm16;
    a.S = S_dev;
    a.out = static_cast<uint8_t*>(blocks);
    a.nvec = n;
    a.hkv = 1;
    a.capacity = 1;
    a.batch = 1;
    set_divisors(a);
    return dispatch_quantize<Src::kRotated>(format, d, a, *cb, stream);
}

int tq_rotate_sketch_query(const tq_layout* L, const tq_codebook* cbk, const float* S_dev, const float* q, float* q_rot,
                           float* q_sketch, hipStream_t stream) {
    using namespace tq;
    int st = check_layout(L);
    if (st != TQ_OK) return st;
    if ((st = check_codebook(cbk, L->k_format, L->head_dim)) != TQ_OK) return st;
    if (!q || !q_rot || !aligned(q, 16) || !aligned(q_rot, 16)) return TQ_ERR_INVALID;
    const bool sketch = L->k_format == TQ_FMT_TQ3K;
    if (sketch && (!S_dev || !q_sketch || !aligned(S_dev, 16) || !aligned(q_sketch, 16))) return TQ_ERR_INVALID;
    const int nvec = L->batch * L->n_q_heads;
    const int d = L->head_dim;
    const int vpb = kWriteThreads / (d / 8);
    const int grid = (nvec + vpb - 1) / vpb;
    const DevCodebook c = to_dev(*cbk);
    if (d == 128) {
        if (sketch)
            hipLaunchKernelGGL((rotate_query_kernel<128, true>), dim3(grid, 128 / sketch_rows_per_wg<128>()),
                               dim3(kWriteThreads), 0, stream, q, q_rot, q_sketch, S_dev, nvec, c);
        else
            hipLaunchKernelGGL((rotate_query_kernel<128, false>), dim3(grid), dim3(kWriteThreads), 0, stream, q, q_rot,
                               nullptr, nullptr, nvec, c);
    } else {
        if (sketch)
            hipLaunchKernelGGL((rotate_query_kernel<256, true>), dim3(grid, 256 / sketch_rows_per_wg<256>()),
                               dim3(kWriteThreads), 0, stream, q, q_rot, q_sketch, S_dev, nvec, c);
        else
            hipLaunchKernelGGL((rotate_query_kernel<256, false>), dim3(grid), dim3(kWriteThreads), 0, stream, q, q_rot,
                               nullptr, nullptr, nvec, c);
    }
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

}  // extern "C"
