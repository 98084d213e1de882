// Host-core driver for the sanitizer build: compiled with g++ and
// -fsanitize=address,undefined together with tq_host.cpp (no device code), it calls
// every host entry point of that file with valid and invalid arguments and checks
// the invariants a caller relies on.  Any sanitizer report or failed check ends the
// process with a nonzero status.  Test infrastructure: built and run by
// tests/test_host_sanitizers.py.

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include "tq_internal.h"

namespace {

int failures = 0;

void check(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "check failed: %s\n", what);
        ++failures;
    }
}

tq_layout layout(int b, int hq, int hkv, int d, int cap, int kf, int vf) {
    tq_layout L;
    std::memset(&L, 0, sizeof(L));
    L.batch = b;
    L.n_q_heads = hq;
    L.n_kv_heads = hkv;
    L.head_dim = d;
    L.capacity = cap;
    L.k_format = kf;
    L.v_format = vf;
    return L;
}

void codebooks() {
    for (int d : {64, 128, 256}) {
        for (int bits = 1; bits <= 4; ++bits) {
            for (int kind : {TQ_CB_QUANTILE_MEAN, TQ_CB_LLOYD_MAX}) {
                tq_codebook cb;
                std::vector<float> S(static_cast<size_t>(d) * d, std::numeric_limits<float>::quiet_NaN());
                const int st = tq_build_codebook(d, bits, kind, 1234 + d, 99, &cb, S.data());
                check(st == TQ_OK, "codebook builds");
                if (st != TQ_OK) continue;
                const int K = 1 << bits;
                check(cb.n_levels == K && cb.head_dim == d && cb.bits == bits, "codebook header");
                for (int k = 0; k < K; ++k) check(cb.centroids[k] == -cb.centroids[K - 1 - k], "odd symmetry");
                for (int k = 0; k + 1 < K; ++k) {
                    check(cb.centroids[k] < cb.centroids[k + 1], "centroids increase");
                    check(cb.centroids[k] < cb.bounds[k] && cb.bounds[k] < cb.centroids[k + 1], "bounds between");
                }
                for (int k = K - 1; k < 16; ++k) check(std::isinf(cb.bounds[k]), "unused bounds +inf");
                double sum = 0.0, sq = 0.0;
                for (float v : S) {
                    check(std::isfinite(v), "S finite");
                    sum += v;
                    sq += static_cast<double>(v) * v;
                }
                const double n = static_cast<double>(S.size());
                check(std::fabs(sum / n) < 6.0 / std::sqrt(n) && std::fabs(sq / n - 1.0) < 0.1, "S ~ N(0, 1)");
                tq_codebook again;
                check(tq_build_codebook(d, bits, kind, 1234 + d, 99, &again, nullptr) == TQ_OK &&
                          std::memcmp(&cb, &again, sizeof(cb)) == 0,
                      "deterministic, S optional");
            }
        }
    }
    tq_codebook cb;
    check(tq_build_codebook(128, 4, 0, 1, 2, nullptr, nullptr) == TQ_ERR_INVALID, "null out");
    check(tq_build_codebook(96, 4, 0, 1, 2, &cb, nullptr) == TQ_ERR_UNSUPPORTED, "head dim");
    check(tq_build_codebook(128, 0, 0, 1, 2, &cb, nullptr) == TQ_ERR_UNSUPPORTED, "bits 0");
    check(tq_build_codebook(128, 5, 0, 1, 2, &cb, nullptr) == TQ_ERR_UNSUPPORTED, "bits 5");
    check(tq_build_codebook(128, 4, 7, 1, 2, &cb, nullptr) == TQ_ERR_UNSUPPORTED, "kind");
    check(tq::check_codebook(nullptr, TQ_FMT_PQ4, 128) == TQ_ERR_INVALID, "null codebook");
    tq_build_codebook(128, 4, 0, 1, 2, &cb, nullptr);
    check(tq::check_codebook(&cb, TQ_FMT_PQ4, 128) == TQ_OK, "PQ4 table");
    check(tq::check_codebook(&cb, TQ_FMT_PQ3, 128) == TQ_ERR_INVALID, "3-bit format, 4-bit table");
    check(tq::check_codebook(&cb, TQ_FMT_PQ4, 256) == TQ_ERR_INVALID, "head dim mismatch");
    check(tq::check_codebook(&cb, TQ_FMT_GQ4V, 256) == TQ_OK, "group formats ignore the table");
}

void sizes_and_layouts() {
    const int fmts[] = {TQ_FMT_PQ4, TQ_FMT_PQ3, TQ_FMT_TQ3K, TQ_FMT_GQ2V, TQ_FMT_GQ4V};
    const size_t want128[] = {68, 56, 52, 48, 80}, want256[] = {136, 112, 100, 96, 160};  // TQ3K: one header
    for (int i = 0; i < 5; ++i) {
        check(tq_vector_bytes(fmts[i], 128) == want128[i], "vector bytes at d 128");
        check(tq_vector_bytes(fmts[i], 256) == want256[i], "vector bytes at d 256");
        check(tq_vector_bytes(fmts[i], 64) == 0 && tq_vector_bytes(fmts[i], 512) == 0, "no other head dims");
    }
    check(tq_vector_bytes(0, 128) == 0 && tq_vector_bytes(6, 128) == 0 && tq_vector_bytes(-1, 128) == 0,
          "unknown formats");
    check(std::strlen(tq_version()) > 0, "version");
    for (int s = 1; s >= -7; --s) check(tq_strerror(s) != nullptr && std::strlen(tq_strerror(s)) > 0, "strerror");

    size_t kb = 0, vb = 0;
    tq_layout L = layout(8, 32, 8, 128, 65536, TQ_FMT_PQ4, TQ_FMT_PQ4);
    check(tq_cache_bytes(&L, &kb, &vb) == TQ_OK && kb == 8ull * 8 * 65536 * 68 && vb == kb, "C4 cache bytes");
    L = layout(1, 40, 8, 128, 30016, TQ_FMT_TQ3K, TQ_FMT_GQ4V);
    check(tq_cache_bytes(&L, &kb, &vb) == TQ_OK && kb == 8ull * 30016 * 52 && vb == 8ull * 30016 * 80,
          "TQ3K / GQ4V cache bytes");
    check(tq_cache_bytes(nullptr, &kb, &vb) == TQ_ERR_INVALID, "null layout");
    check(tq_cache_bytes(&L, nullptr, &vb) == TQ_ERR_INVALID, "null output");
    const tq_layout bad[] = {
        layout(0, 4, 1, 128, 64, TQ_FMT_PQ4, TQ_FMT_PQ4),    layout(1, 5, 2, 128, 64, TQ_FMT_PQ4, TQ_FMT_PQ4),
        layout(1, 4, 1, 128, 65, TQ_FMT_PQ4, TQ_FMT_PQ4),    layout(1, 4, 0, 128, 64, TQ_FMT_PQ4, TQ_FMT_PQ4),
        layout(1, 4, 1, 128, -64, TQ_FMT_PQ4, TQ_FMT_PQ4),   layout(-1, 4, 1, 128, 64, TQ_FMT_PQ4, TQ_FMT_PQ4),
    };
    for (const tq_layout& b : bad) check(tq_cache_bytes(&b, &kb, &vb) == TQ_ERR_INVALID, "bad shape");
    tq_layout r = layout(1, 4, 1, 128, 64, TQ_FMT_PQ4, TQ_FMT_PQ4);
    r.reserved = 1;
    check(tq_cache_bytes(&r, &kb, &vb) == TQ_ERR_INVALID, "reserved field");
    const tq_layout unsup[] = {
        layout(1, 4, 1, 64, 64, TQ_FMT_PQ4, TQ_FMT_PQ4),     layout(1, 4, 1, 128, 64, TQ_FMT_PQ4, TQ_FMT_PQ3),
        layout(1, 4, 1, 128, 64, TQ_FMT_GQ2V, TQ_FMT_GQ2V),  layout(1, 4, 1, 128, 64, TQ_FMT_TQ3K, TQ_FMT_PQ4),
        layout(1, 4, 1, 128, 64, 9, TQ_FMT_PQ4),
    };
    for (const tq_layout& u : unsup) check(tq_cache_bytes(&u, &kb, &vb) == TQ_ERR_UNSUPPORTED, "unsupported");
    const tq_layout huge = layout(65536, 64, 64, 128, 1 << 20, TQ_FMT_PQ4, TQ_FMT_PQ4);
    check(tq_cache_bytes(&huge, &kb, &vb) == TQ_ERR_RANGE, "more vectors than 31 bits index");

    // workspace regions: 256-byte aligned, in order, large enough
    for (int splits : {1, 3, 16, 257}) {
        const tq_layout w = layout(3, 15, 5, 256, 1024, TQ_FMT_PQ4, TQ_FMT_PQ4);
        const tq::WsLayout ws = tq::ws_layout(w, splits);
        const size_t recs = 3ull * 15 * splits;
        check(ws.acc % 256 == 0 && ws.cnt % 256 == 0 && ws.total % 256 == 0, "aligned regions");
        check(ws.acc >= recs * 8 && ws.cnt - ws.acc >= recs * 256 * 4 && ws.total - ws.cnt >= 3ull * 5 * 4,
              "region sizes");
    }
    check(tq::is_rotated(TQ_FMT_PQ4) && tq::is_rotated(TQ_FMT_PQ3) && tq::is_rotated(TQ_FMT_TQ3K) &&
              !tq::is_rotated(TQ_FMT_GQ2V) && !tq::is_rotated(TQ_FMT_GQ4V),
          "rotated formats");
    check(tq::is_group_quant(TQ_FMT_GQ2V) && tq::is_group_quant(TQ_FMT_GQ4V) && !tq::is_group_quant(TQ_FMT_PQ4),
          "group formats");
    check(tq::format_bits(TQ_FMT_PQ4) == 4 && tq::format_bits(TQ_FMT_PQ3) == 3 && tq::format_bits(TQ_FMT_TQ3K) == 2 &&
              tq::format_bits(TQ_FMT_GQ2V) == 0,
          "table bits");
    alignas(16) unsigned char buf[32];
    check(tq::aligned(buf, 16) && !tq::aligned(buf + 4, 16) && tq::aligned(buf + 4, 4), "alignment test");
}

}  // namespace

int main() {
    codebooks();
    sizes_and_layouts();
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("host core: all checks passed\n");
    return 0;
}
