// Host core of libtq: codebook construction, the splitmix64 stream, the
// Box-Muller QJL matrix, layout arithmetic, validation and error text.
// Plain C++17 with libm; no device code.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "tq_internal.h"

namespace {

// ---------------------------------------------------------------------------
// Normal distribution helpers (double precision)

constexpr double kInvSqrt2Pi = 0.39894228040143267794;

double pdf(double z) {
    if (!std::isfinite(z)) return 0.0;
    return std::exp(-0.5 * z * z) * kInvSqrt2Pi;
}

double cdf(double z) {
    if (z == -INFINITY) return 0.0;
    if (z == INFINITY) return 1.0;
    return 0.5 * std::erfc(-z / std::sqrt(2.0));
}

// Inverse of the standard normal CDF: P. J. Acklam's rational approximation
// (relative error below 1.2e-9) refined by two Halley steps on erfc, which
// brings it to full double precision.
double inv_cdf(double p) {
    if (p <= 0.0) return -INFINITY;
    if (p >= 1.0) return INFINITY;
    static const double a[] = {-3.969683028665376e+01, 2.209460984245205e+02, -2.759285104469687e+02,
                               1.383577518672690e+02, -3.066479806614716e+01, 2.506628277459239e+00};
    static const double b[] = {-5.447609879822406e+01, 1.615858368580409e+02, -1.556989798598866e+02,
                               6.680131188771972e+01, -1.328068155288572e+01};
    static const double c[] = {-7.784894002430293e-03, -3.223964580411365e-01, -2.400758277161838e+00,
                               -2.549732539343734e+00, 4.374664141464968e+00, 2.938163982698783e+00};
    static const double d[] = {7.784695709041462e-03, 3.224671290700398e-01, 2.445134137142996e+00,
                               3.754408661907416e+00};
    const double plow = 0.02425, phigh = 1 - plow;
    double x;
    if (p < plow) {
        double q = std::sqrt(-2 * std::log(p));
        x = (((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
            ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1);
    } else if (p <= phigh) {
        double q = p - 0.5, r = q * q;
        x = (((((a[0] * r + a[1]) * r + a[2]) * r + a[3]) * r + a[4]) * r + a[5]) * q /
            (((((b[0] * r + b[1]) * r + b[2]) * r + b[3]) * r + b[4]) * r + 1);
    } else {
        double q = std::sqrt(-2 * std::log(1 - p));
        x = -(((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
            ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1);
    }
    for (int it = 0; it < 2; ++it) {
        double e = cdf(x) - p;
        double u = e * std::sqrt(2 * M_PI) * std::exp(0.5 * x * x);
        x = x - u / (1 + 0.5 * x * u);
    }
    return x;
}

// Make a standardized table exactly odd-symmetric: c_k = (c_k - c_{K-1-k}) / 2.
void symmetrize(std::vector<double>& c) {
    const int K = static_cast<int>(c.size());
    std::vector<double> o(K);
    for (int k = 0; k < K; ++k) o[k] = 0.5 * (c[k] - c[K - 1 - k]);
    c = o;
}

// Conditional means of N(0,1) over the K equal-probability intervals.
std::vector<double> quantile_mean_std(int K) {
    std::vector<double> z(K + 1);
    for (int k = 0; k <= K; ++k) z[k] = inv_cdf(static_cast<double>(k) / K);
    std::vector<double> c(K);
    for (int k = 0; k < K; ++k) c[k] = K * (pdf(z[k]) - pdf(z[k + 1]));
    symmetrize(c);
    return c;
}

// Fixed point of the Lloyd conditions for N(0,1), started from the quantile means.
std::vector<double> lloyd_max_std(int K) {
    std::vector<double> c = quantile_mean_std(K);
    std::vector<double> e(K + 1), n(K);
    for (int it = 0; it < 200000; ++it) {
        e[0] = -INFINITY;
        e[K] = INFINITY;
        for (int k = 1; k < K; ++k) e[k] = 0.5 * (c[k - 1] + c[k]);
        for (int k = 0; k < K; ++k) n[k] = (pdf(e[k]) - pdf(e[k + 1])) / (cdf(e[k + 1]) - cdf(e[k]));
        symmetrize(n);
        double delta = 0;
        for (int k = 0; k < K; ++k) delta = std::fmax(delta, std::fabs(n[k] - c[k]));
        c = n;
        if (delta < 1e-13) break;
    }
    return c;
}

// splitmix64 (Steele, Lea and Flood 2014): output i of the stream seeded with
// `seed` is mix(seed + (i + 1) * golden_gamma).
struct SplitMix64 {
    uint64_t state;
    uint64_t next() {
        state += 0x9E3779B97F4A7C15ull;
        uint64_t z = state;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
};

double unit_open(uint64_t x) { return (static_cast<double>(x >> 11) + 0.5) * 0x1.0p-53; }

}  // namespace

namespace tq {

size_t vector_bytes(int format, int d) {
    if (d != 128 && d != 256) return 0;
    switch (format) {
        case TQ_FMT_PQ4: return static_cast<size_t>(68) * (d / 128);
        case TQ_FMT_PQ3: return static_cast<size_t>(14) * (d / 32);
        case TQ_FMT_TQ3K: return static_cast<size_t>(4 + d / 4 + d / 8);
        case TQ_FMT_GQ2V: return static_cast<size_t>(12) * (d / kGroup);
        case TQ_FMT_GQ4V: return static_cast<size_t>(20) * (d / kGroup);
        default: return 0;
    }
}

bool is_rotated(int format) { return format == TQ_FMT_PQ4 || format == TQ_FMT_PQ3 || format == TQ_FMT_TQ3K; }

bool is_group_quant(int format) { return format == TQ_FMT_GQ2V || format == TQ_FMT_GQ4V; }

int format_bits(int format) {
    switch (format) {
        case TQ_FMT_PQ4: return 4;
        case TQ_FMT_PQ3: return 3;
        case TQ_FMT_TQ3K: return 2;
        default: return 0;
    }
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A bound on how far past a stream's end a decode kernel's tile requests reach (a workgroup's
// first tiles and the tiles it requests ahead; they read zeros there): under a thousand tokens.
constexpr double kStreamSlack = 4096.0;

int check_layout(const tq_layout* L) {
    if (!L) return TQ_ERR_INVALID;
    if (L->batch <= 0 || L->n_q_heads <= 0 || L->n_kv_heads <= 0 || L->capacity <= 0 || L->reserved != 0)
        return TQ_ERR_INVALID;
    if (L->n_q_heads % L->n_kv_heads) return TQ_ERR_INVALID;
    if (L->capacity % kTile) return TQ_ERR_INVALID;
    if (L->head_dim != 128 && L->head_dim != 256) return TQ_ERR_UNSUPPORTED;
    const int kf = L->k_format, vf = L->v_format;
    const bool ok = (kf == TQ_FMT_PQ4 && vf == TQ_FMT_PQ4) || (kf == TQ_FMT_PQ3 && vf == TQ_FMT_PQ3) ||
                    (kf == TQ_FMT_PQ3 && vf == TQ_FMT_PQ4) || (kf == TQ_FMT_TQ3K && vf == TQ_FMT_GQ2V) ||
                    (kf == TQ_FMT_TQ3K && vf == TQ_FMT_GQ4V);
    if (!ok) return TQ_ERR_UNSUPPORTED;
    // every byte offset of a cache must fit in 63 bits and every index in 31
    const double vecs = static_cast<double>(L->batch) * L->n_kv_heads * L->capacity;
    if (vecs > 2147483647.0) return TQ_ERR_RANGE;
    // the decode kernels address one (b, kv-head) stream with 32-bit byte offsets, including
    // the tiles they request past its end (fewer than kStreamSlack tokens)
    const double vb = static_cast<double>(std::max(vector_bytes(kf, L->head_dim), vector_bytes(vf, L->head_dim)));
    if ((static_cast<double>(L->capacity) + kStreamSlack) * vb > 2147483647.0) return TQ_ERR_RANGE;
    return TQ_OK;
}

int check_codebook(const tq_codebook* cb, int format, int d) {
    if (!cb) return TQ_ERR_INVALID;
    if (is_group_quant(format)) return TQ_OK;  // no table: scale and zero per group
    if (cb->head_dim != d) return TQ_ERR_INVALID;
    if (cb->bits != format_bits(format) || cb->n_levels != (1 << cb->bits)) return TQ_ERR_INVALID;
    return TQ_OK;
}

}  // namespace tq

extern "C" {

const char* tq_version(void) { return "libtq 0.1.0 (gfx950)"; }

const char* tq_strerror(int status) {
    switch (status) {
        case TQ_OK: return "ok";
        case TQ_ERR_INVALID: return "invalid argument (null pointer, bad shape or misaligned buffer)";
        case TQ_ERR_UNSUPPORTED: return "unsupported head dim, bit width or format pair";
        case TQ_ERR_WORKSPACE: return "workspace smaller than required";
        case TQ_ERR_RANGE: return "size exceeds what the call can address";
        case TQ_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

int tq_build_codebook(int head_dim, int bits, int kind, uint64_t rot_seed, uint64_t qjl_seed, tq_codebook* out,
                      float* qjl_S) {
    if (!out) return TQ_ERR_INVALID;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256) return TQ_ERR_UNSUPPORTED;
    if (bits < 1 || bits > 4) return TQ_ERR_UNSUPPORTED;
    if (kind != TQ_CB_QUANTILE_MEAN && kind != TQ_CB_LLOYD_MAX) return TQ_ERR_UNSUPPORTED;
    const int K = 1 << bits;
    std::vector<double> c = kind == TQ_CB_QUANTILE_MEAN ? quantile_mean_std(K) : lloyd_max_std(K);
    const double sigma = 1.0 / std::sqrt(static_cast<double>(head_dim));
    tq_codebook cb;
    std::memset(&cb, 0, sizeof(cb));
    cb.head_dim = head_dim;
    cb.bits = bits;
    cb.kind = kind;
    cb.n_levels = K;
    cb.rot_seed = rot_seed;
    cb.qjl_seed = qjl_seed;
    std::vector<double> cs(K);
    for (int k = 0; k < K; ++k) cs[k] = sigma * c[k];
    for (int k = 0; k < K; ++k) cb.centroids[k] = static_cast<float>(cs[k]);
    for (int k = 0; k + 1 < K; ++k) cb.bounds[k] = static_cast<float>(0.5 * (cs[k] + cs[k + 1]));
    for (int k = K - 1; k < 16; ++k) cb.bounds[k] = INFINITY;  // unused slots never count
    SplitMix64 rs{rot_seed};
    for (int j = 0; j < head_dim; ++j)
        if (rs.next() >> 63) cb.sign_bits[j >> 5] |= 1u << (j & 31);
    if (qjl_S) {
        SplitMix64 qs{qjl_seed};
        const int n = head_dim * head_dim;
        for (int t = 0; t < n / 2; ++t) {
            const double u1 = unit_open(qs.next());
            const double u2 = unit_open(qs.next());
            const double r = std::sqrt(-2.0 * std::log(u1));
            const double a = 2.0 * M_PI * u2;
            qjl_S[2 * t] = static_cast<float>(r * std::cos(a));
            qjl_S[2 * t + 1] = static_cast<float>(r * std::sin(a));
        }
    }
    *out = cb;
    return TQ_OK;
}

size_t tq_vector_bytes(int format, int head_dim) { return tq::vector_bytes(format, head_dim); }

int tq_cache_bytes(const tq_layout* L, size_t* k_bytes, size_t* v_bytes) {
    const int st = tq::check_layout(L);
    if (st != TQ_OK) return st;
    if (!k_bytes || !v_bytes) return TQ_ERR_INVALID;
    const size_t vecs = static_cast<size_t>(L->batch) * L->n_kv_heads * L->capacity;
    *k_bytes = vecs * tq::vector_bytes(L->k_format, L->head_dim);
    *v_bytes = vecs * tq::vector_bytes(L->v_format, L->head_dim);
    return TQ_OK;
}

}  // extern "C"
