// Internal declarations shared by the host core and the HIP translation
// units of libtq.  Not part of the public ABI (see include/tq.h).
#pragma once

#include <cstddef>
#include <cstdint>

#include "tq.h"

namespace tq {

constexpr int kGroup = 32;        // GQ2V channels per group
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

size_t vector_bytes(int format, int d);
bool is_rotated(int format);
int format_bits(int format);  // code bits per coordinate a format stores in its table
int check_layout(const tq_layout* L);
int check_codebook(const tq_codebook* cb, int format, int d);
bool aligned(const void* p, size_t a);

}  // namespace tq
