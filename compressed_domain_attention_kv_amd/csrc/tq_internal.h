// Internal declarations shared by the host core and the HIP translation
// units of libtq.  Not part of the public ABI (see include/tq.h).
#pragma once

#include <cstddef>
#include <cstdint>

#include "tq.h"

namespace tq {

constexpr int kGroup = 32;        // GQ2V / GQ4V channels per group
constexpr int kTile = 64;         // tokens per wavefront tile in the decode kernel
constexpr int kWaves = 4;         // wavefronts per decode workgroup
constexpr int kSplitQuantum = kTile * kWaves;
constexpr float kFp16Max = 65504.0f;
constexpr int kRingCapMax = TQ_RING_CAP_MAX;  // capture ring slots per stream

// Codebook data a kernel needs, passed by value as a kernel argument.
struct DevCodebook {
    float centroids[16];
    float bounds[16];
    uint32_t sign_bits[8];
};

inline DevCodebook to_dev(const tq_codebook& cb) {
    DevCodebook d{};
    for (int i = 0; i < 16; ++i) {
        d.centroids[i] = cb.centroids[i];
        d.bounds[i] = cb.bounds[i];
    }
    for (int i = 0; i < 8; ++i) d.sign_bits[i] = cb.sign_bits[i];
    return d;
}

// Byte layout of a decode workspace with `splits` records per (b, query head) row:
//   [0, acc)      float2 ml[B][Hq][splits]          (m, l) of every split record
//   [acc, cnt)    float  acc[B][Hq][splits][d]      unnormalized value sums
//   [cnt, total)  uint32 arrivals[B][Hkv]           workgroups of a stream done so far
// Each region starts on a 256-byte boundary.  The arrival counters serve the decodes
// that merge the records in the same launch: the last workgroup of a stream to arrive
// merges it and sets its counter back to zero, so the counters are zero between calls
// once they have been cleared after allocation.
struct WsLayout {
    size_t acc, cnt, total;
};

constexpr size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline WsLayout ws_layout(const tq_layout& L, int splits) {
    const size_t recs = static_cast<size_t>(L.batch) * L.n_q_heads * splits;
    WsLayout w{};
    w.acc = round_up(recs * 8, 256);
    w.cnt = w.acc + round_up(recs * static_cast<size_t>(L.head_dim) * 4, 256);
    w.total = w.cnt + round_up(static_cast<size_t>(L.batch) * L.n_kv_heads * 4, 256);
    return w;
}

// The capture ring a hybrid read attends over besides the compressed records.
struct RingView {
    const float* q_rot;
    const void* k_ring;
    const void* v_ring;
    const int32_t* comp_lens;
    const int32_t* ring_lens;
    int ring_cap;
};

// Merge the `splits` records of every (b, query head) row of the decode workspace,
// and the capture ring when one is given; normalize, rotate back (tq_combine.hip).
int combine(const tq_layout* L, const tq_codebook* cbk, const tq_codebook& cbv, int splits, const void* ws,
            float* out, hipStream_t stream, const RingView* ring = nullptr);

// Zero n words of device memory with a fill kernel (graph-capturable, unlike a memset node).
int clear_words(uint32_t* p, size_t n, hipStream_t stream);

size_t vector_bytes(int format, int d);
bool is_rotated(int format);
bool is_group_quant(int format);  // GQ2V, GQ4V: per-group scale and zero, no rotation
int format_bits(int format);  // code bits per coordinate a format stores in its table
int check_layout(const tq_layout* L);
int check_codebook(const tq_codebook* cb, int format, int d);
bool aligned(const void* p, size_t a);

}  // namespace tq
