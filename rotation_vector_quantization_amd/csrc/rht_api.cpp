// rht_api.cpp -- the C ABI of librht (declared in include/rht.h): argument
// validation, the host-side codebook and rotation signs, and kernel dispatch.
//
// The codebook is the N(0,1) Lloyd-Max quantizer named on the web page
// "Random-rotation quantization" ("History", EDEN item: computed once for the
// standard normal; 1 bit +-sqrt(2/pi), 2 bits +-0.453, +-1.510).  It is solved
// here on the positive half-line (the density is even, so the quantizer is
// antisymmetric with 0 as its middle threshold), in double, then rounded to
// fp32 for the kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/rht.h"
#include "rht_internal.h"

namespace rht {
namespace {

struct FloatBook {
    float lev[16];
    float thr[16];
};

FloatBook g_books[5];
std::once_flag g_books_once;

// Upper-tail probability and density of N(0,1).
double upper_tail(double t) { return std::isinf(t) ? 0.0 : 0.5 * std::erfc(t / std::sqrt(2.0)); }
double density(double t) { return std::isinf(t) ? 0.0 : std::exp(-0.5 * t * t) / std::sqrt(2.0 * M_PI); }

// Positive half of the 2^bits-level Lloyd-Max quantizer: h = 2^(bits-1)
// levels p[0] < ... < p[h-1] with cells [b_j, b_{j+1}), b_0 = 0, b_h = inf,
// b_j = (p[j-1] + p[j]) / 2.  Each level is its cell's conditional mean,
// (density(b_j) - density(b_{j+1})) / (tail(b_j) - tail(b_{j+1})).
void solve_half(int bits, double *p) {
    const int h = 1 << (bits - 1);
    for (int j = 0; j < h; ++j) p[j] = (j + 0.5) * 2.5 / h;
    for (int it = 0; it < 200000; ++it) {
        double edges[9];
        edges[0] = 0.0;
        for (int j = 1; j < h; ++j) edges[j] = 0.5 * (p[j - 1] + p[j]);
        edges[h] = INFINITY;
        double change = 0.0;
        for (int j = 0; j < h; ++j) {
            const double mass = upper_tail(edges[j]) - upper_tail(edges[j + 1]);
            const double c = (density(edges[j]) - density(edges[j + 1])) / mass;
            change = std::fmax(change, std::fabs(c - p[j]));
            p[j] = c;
        }
        if (change < 1e-15) break;
    }
}

void fill_book(FloatBook &fb, int bits, const double *p);

void build_books() {
    for (int bits = 1; bits <= 4; ++bits) {
        const int h = 1 << (bits - 1), K = 2 * h;
        double p[8];
        solve_half(bits, p);
        fill_book(g_books[bits], bits, p);
        (void)h;
        (void)K;
    }
}

// Exact finite-d codebook ("Why rotation works": a coordinate t of a
// uniformly rotated unit vector follows a Beta law, (1 + t)/2 ~
// Beta((d-1)/2, (d-1)/2); the codebook is the Lloyd-Max quantizer of
// y = sqrt(d) t).  Solved on the positive half-line like the N(0,1) one, with
// cell masses from the regularized incomplete beta function and cell first
// moments in closed form:
//   integral of y f(y) over [y1, y2) = sqrt(d) / ((d-1) B(1/2, (d-1)/2))
//       * ((1 - t1^2)^((d-1)/2) - (1 - t2^2)^((d-1)/2)),  t = y / sqrt(d).

// Continued fraction of I_x(a, b) (Abramowitz and Stegun 26.5.8), evaluated
// with the modified Lentz method; accurate for x < (a + 1) / (a + b + 2).
double beta_cf(double a, double b, double x) {
    const double tiny = 1e-300;
    double c = 1.0, dd = 1.0 - (a + b) * x / (a + 1.0);
    if (std::fabs(dd) < tiny) dd = tiny;
    dd = 1.0 / dd;
    double f = dd;
    for (int m = 1; m < 10000; ++m) {
        // even step: m (b - m) x / ((a + 2m - 1)(a + 2m))
        double num = m * (b - m) * x / ((a + 2.0 * m - 1.0) * (a + 2.0 * m));
        dd = 1.0 + num * dd;
        c = 1.0 + num / c;
        if (std::fabs(dd) < tiny) dd = tiny;
        if (std::fabs(c) < tiny) c = tiny;
        dd = 1.0 / dd;
        f *= dd * c;
        // odd step: -(a + m)(a + b + m) x / ((a + 2m)(a + 2m + 1))
        num = -(a + m) * (a + b + m) * x / ((a + 2.0 * m) * (a + 2.0 * m + 1.0));
        dd = 1.0 + num * dd;
        c = 1.0 + num / c;
        if (std::fabs(dd) < tiny) dd = tiny;
        if (std::fabs(c) < tiny) c = tiny;
        dd = 1.0 / dd;
        const double step = dd * c;
        f *= step;
        if (std::fabs(step - 1.0) < 1e-16) break;
    }
    return f;
}

// Regularized incomplete beta I_x(a, a) for 0 <= x <= 1/2 (symmetric law).
double inc_beta_sym(double a, double x) {
    if (x <= 0.0) return 0.0;
    const double lnpre = a * std::log(x) + a * std::log1p(-x) - std::log(a) -
                         (2.0 * std::lgamma(a) - std::lgamma(2.0 * a));
    return std::exp(lnpre) * beta_cf(a, a, x);
}

// P(Y >= y) for y >= 0 under the finite-d law.
double beta_upper_tail(double y, int d) {
    const double rd = std::sqrt((double)d);
    if (y >= rd) return 0.0;
    return inc_beta_sym(0.5 * (d - 1), 0.5 * (1.0 - y / rd));
}

// First-moment kernel (1 - t^2)^((d-1)/2) at y (0 beyond the support).
double beta_moment_kernel(double y, int d) {
    const double t = y / std::sqrt((double)d);
    return t >= 1.0 ? 0.0 : std::exp(0.5 * (d - 1) * std::log1p(-t * t));
}

void solve_half_beta(int bits, int d, double *p) {
    const int h = 1 << (bits - 1);
    const double rd = std::sqrt((double)d);
    // sqrt(d) / ((d-1) B(1/2, (d-1)/2))
    const double mk = rd / (d - 1.0) *
                      std::exp(std::lgamma(0.5 * d) - std::lgamma(0.5) - std::lgamma(0.5 * (d - 1)));
    for (int j = 0; j < h; ++j) p[j] = std::fmin((j + 0.5) * 2.5 / h, 0.9 * rd);
    for (int it = 0; it < 200000; ++it) {
        double edges[9];
        edges[0] = 0.0;
        for (int j = 1; j < h; ++j) edges[j] = 0.5 * (p[j - 1] + p[j]);
        edges[h] = rd;
        double change = 0.0;
        for (int j = 0; j < h; ++j) {
            const double mass = beta_upper_tail(edges[j], d) - beta_upper_tail(edges[j + 1], d);
            const double c = mk * (beta_moment_kernel(edges[j], d) - beta_moment_kernel(edges[j + 1], d)) / mass;
            change = std::fmax(change, std::fabs(c - p[j]));
            p[j] = c;
        }
        if (change < 1e-14) break;
    }
}

void fill_book(FloatBook &fb, int bits, const double *p) {
    const int h = 1 << (bits - 1);
    std::memset(&fb, 0, sizeof(fb));
    for (int j = 0; j < h; ++j) {
        fb.lev[h + j] = (float)p[j];
        fb.lev[h - 1 - j] = (float)-p[j];
    }
    fb.thr[h - 1] = 0.0f;
    for (int j = 1; j < h; ++j) {
        const float t = (float)(0.5 * (p[j - 1] + p[j]));
        fb.thr[h - 1 + j] = t;
        fb.thr[h - 1 - j] = -t;
    }
}

constexpr int kLogMaxD = 12;
FloatBook g_beta[5][kLogMaxD + 1];
std::once_flag g_beta_once[5][kLogMaxD + 1];

// The finite-d codebook for a supported (bits, d); computed once.
const FloatBook &beta_book(int bits, int d) {
    int lg = 0;
    while ((1 << lg) < d) ++lg;
    std::call_once(g_beta_once[bits][lg], [bits, d, lg] {
        double p[8];
        solve_half_beta(bits, d, p);
        fill_book(g_beta[bits][lg], bits, p);
    });
    return g_beta[bits][lg];
}

const FloatBook &book(int bits) {
    std::call_once(g_books_once, build_books);
    return g_books[bits];
}

// Sign i of D: top bit of the i-th SplitMix64 output (Steele, Lea, Flood 2014)
// from state `seed`; 1 means -1.  The generator's state after i + 1 steps is
// seed + (i + 1) * 0x9E3779B97F4A7C15 (mod 2^64), so each output stands alone.
uint32_t sign_bit(uint64_t seed, int i) {
    uint64_t z = seed + (uint64_t)(i + 1) * 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return (uint32_t)(z >> 63);
}

// The signs of D as bit words, bit i % 32 of word i / 32.
void sign_words(uint64_t seed, int d, uint32_t *words) {
    std::memset(words, 0, sizeof(uint32_t) * (size_t)((d + 31) / 32));
    for (int i = 0; i < d; ++i) words[i >> 5] |= sign_bit(seed, i) << (i & 31);
}

bool pow2_dim(int32_t d) { return d >= kMinD && d <= kMaxD && (d & (d - 1)) == 0; }
bool aligned(const void *p) { return ((uintptr_t)p & 15u) == 0; }

rht_status launched(hipError_t e) { return e == hipSuccess ? RHT_OK : RHT_E_DEVICE; }

// Key chunks per head for attention: enough (head, chunk) wavefronts to fill
// the chip once (256 CUs x 12 resident waves), never more chunks than 32-key
// tiles.  A fixed count keeps the workspace size independent of the device.
int64_t attention_chunks(int64_t heads, int64_t n) {
    const int64_t tiles = (n + 31) / 32;
    int64_t c = (3072 + heads - 1) / heads;
    if (c > tiles) c = tiles;
    if (c > 1024) c = 1024;
    return c < 1 ? 1 : c;
}

bool attention_args_ok(int64_t heads, int32_t m, int64_t n) {
    return heads >= 0 && m >= 1 && m <= kAttnMaxQueries && heads <= kAttnMaxRows / m &&
           (heads == 0 || (n >= 1 && n <= kAttnMaxKeys));
}

std::atomic<int> g_cu[64];

}  // namespace

bool hadamard_on_mfma() {
    static const bool v = [] {
        const char *e = std::getenv("RHT_HADAMARD");
        return !(e && std::strcmp(e, "valu") == 0);
    }();
    return v;
}

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = g_cu[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        g_cu[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

}  // namespace rht

using namespace rht;

extern "C" {

int32_t rht_abi_version(void) { return RHT_ABI_VERSION; }

const char *rht_status_str(rht_status s) {
    switch (s) {
    case RHT_OK: return "ok";
    case RHT_E_NULL: return "null pointer";
    case RHT_E_DIM: return "unsupported dimension d";
    case RHT_E_BITS: return "unsupported bit width";
    case RHT_E_DTYPE: return "unknown element type";
    case RHT_E_MODE: return "unknown mode or mode/bits mismatch";
    case RHT_E_ALIGN: return "device pointer not 16-byte aligned";
    case RHT_E_COUNT: return "negative count or m out of range";
    case RHT_E_DEVICE: return "HIP runtime error";
    case RHT_E_WORKSPACE: return "workspace too small";
    }
    return "unknown status";
}

rht_status rht_codebook(int32_t bits, float *levels, float *thresholds) {
    if (bits < 1 || bits > 4) return RHT_E_BITS;
    const FloatBook &b = book(bits);
    const int K = 1 << bits;
    if (levels) std::memcpy(levels, b.lev, sizeof(float) * (size_t)K);
    if (thresholds) std::memcpy(thresholds, b.thr, sizeof(float) * (size_t)(K - 1));
    return RHT_OK;
}

rht_status rht_codebook_beta(int32_t bits, int32_t d, float *levels, float *thresholds) {
    if (bits < 1 || bits > 4) return RHT_E_BITS;
    if (!pow2_dim(d)) return RHT_E_DIM;
    const FloatBook &b = beta_book(bits, d);
    if (levels) std::memcpy(levels, b.lev, sizeof(float) * (1u << bits));
    if (thresholds) std::memcpy(thresholds, b.thr, sizeof(float) * ((1u << bits) - 1));
    return RHT_OK;
}

rht_status rht_signs(uint64_t seed, int32_t d, int8_t *signs) {
    if (!signs) return RHT_E_NULL;
    if (d < 1 || d > (1 << 20)) return RHT_E_DIM;
    for (int i = 0; i < d; ++i) signs[i] = sign_bit(seed, i) ? (int8_t)-1 : (int8_t)1;
    return RHT_OK;
}

rht_status rht_quantize(const void *x, rht_dtype xt, int64_t n, int32_t d, int32_t bits,
                        rht_mode mode, uint64_t seed, uint8_t *codes, float *scale, void *stream) {
    if (n < 0) return RHT_E_COUNT;
    if (!pow2_dim(d)) return RHT_E_DIM;
    if (bits < 1 || bits > 4) return RHT_E_BITS;
    if (mode != RHT_SCALE_NORM && mode != RHT_SCALE_SIGN_BIASED && mode != RHT_SCALE_SIGN_UNBIASED &&
        mode != RHT_SCALE_EDEN && mode != RHT_SCALE_NORM_BETA)
        return RHT_E_MODE;
    if ((mode == RHT_SCALE_SIGN_BIASED || mode == RHT_SCALE_SIGN_UNBIASED) && bits != 1) return RHT_E_MODE;
    if (xt != RHT_F32 && xt != RHT_F16) return RHT_E_DTYPE;
    if (n == 0) return RHT_OK;
    if (!x || !codes || !scale) return RHT_E_NULL;
    if (!aligned(x) || !aligned(codes) || !aligned(scale)) return RHT_E_ALIGN;

    QuantArgs a;
    std::memset(&a, 0, sizeof(a));
    a.x = x;
    a.codes = codes;
    a.scale = scale;
    a.n = n;
    const FloatBook &b = mode == RHT_SCALE_NORM_BETA ? beta_book(bits, d) : book(bits);
    std::memcpy(a.lev, b.lev, sizeof(a.lev));
    std::memcpy(a.thr, b.thr, sizeof(a.thr));
    sign_words(seed, d, a.dsign);
    const Kind kind = (mode == RHT_SCALE_NORM || mode == RHT_SCALE_NORM_BETA) ? kMse
                      : mode == RHT_SCALE_EDEN ? kEden
                      : mode == RHT_SCALE_SIGN_BIASED ? kDriveBiased : kDriveUnbiased;
    return launched(launch_quantize(d, xt == RHT_F16, bits, kind, a, (hipStream_t)stream));
}

rht_status rht_dequantize(const uint8_t *codes, const float *scale, int64_t n, int32_t d,
                          int32_t bits, rht_mode mode, uint64_t seed, void *y, rht_dtype yt,
                          void *stream) {
    if (n < 0) return RHT_E_COUNT;
    if (!pow2_dim(d)) return RHT_E_DIM;
    if (bits < 1 || bits > 4) return RHT_E_BITS;
    if (mode != RHT_SCALE_NORM && mode != RHT_SCALE_SIGN_BIASED && mode != RHT_SCALE_SIGN_UNBIASED &&
        mode != RHT_SCALE_EDEN && mode != RHT_SCALE_NORM_BETA)
        return RHT_E_MODE;
    if ((mode == RHT_SCALE_SIGN_BIASED || mode == RHT_SCALE_SIGN_UNBIASED) && bits != 1) return RHT_E_MODE;
    if (yt != RHT_F32 && yt != RHT_F16) return RHT_E_DTYPE;
    if (n == 0) return RHT_OK;
    if (!codes || !scale || !y) return RHT_E_NULL;
    if (!aligned(codes) || !aligned(scale) || !aligned(y)) return RHT_E_ALIGN;

    DequantArgs a;
    std::memset(&a, 0, sizeof(a));
    a.codes = codes;
    a.scale = scale;
    a.y = y;
    a.n = n;
    std::memcpy(a.lev, (mode == RHT_SCALE_NORM_BETA ? beta_book(bits, d) : book(bits)).lev, sizeof(a.lev));
    sign_words(seed, d, a.dsign);
    // an EDEN scale decodes exactly like ||x||: x^ = D H (c * scale / d)
    const Kind kind = (mode == RHT_SCALE_NORM || mode == RHT_SCALE_EDEN || mode == RHT_SCALE_NORM_BETA) ? kMse
                      : mode == RHT_SCALE_SIGN_BIASED ? kDriveBiased : kDriveUnbiased;
    return launched(launch_dequantize(d, yt == RHT_F16, bits, kind, a, (hipStream_t)stream));
}

rht_status rht_residual_quantize(const void *x, rht_dtype xt, int64_t n, int32_t d, int32_t bits,
                                 uint64_t seed, uint8_t *codes, uint8_t *signs, float *norms,
                                 float *res_scale, void *stream) {
    if (n < 0) return RHT_E_COUNT;
    if (!pow2_dim(d)) return RHT_E_DIM;
    if (bits < 2 || bits > 4) return RHT_E_BITS;
    if (xt != RHT_F32 && xt != RHT_F16) return RHT_E_DTYPE;
    if (n == 0) return RHT_OK;
    if (!x || !codes || !signs || !norms || !res_scale) return RHT_E_NULL;
    if (!aligned(x) || !aligned(codes) || !aligned(signs) || !aligned(norms) || !aligned(res_scale))
        return RHT_E_ALIGN;

    QuantArgs a;
    std::memset(&a, 0, sizeof(a));
    a.x = x;
    a.codes = codes;
    a.signs = signs;
    a.scale = norms;
    a.res_scale = res_scale;
    a.n = n;
    const FloatBook &b = book(bits - 1);
    std::memcpy(a.lev, b.lev, sizeof(a.lev));
    std::memcpy(a.thr, b.thr, sizeof(a.thr));
    sign_words(seed, d, a.dsign);
    return launched(launch_quantize(d, xt == RHT_F16, bits, kResidual, a, (hipStream_t)stream));
}

rht_status rht_residual_dequantize(const uint8_t *codes, const uint8_t *signs, const float *norms,
                                   const float *res_scale, int64_t n, int32_t d, int32_t bits,
                                   uint64_t seed, void *y, rht_dtype yt, void *stream) {
    if (n < 0) return RHT_E_COUNT;
    if (!pow2_dim(d)) return RHT_E_DIM;
    if (bits < 2 || bits > 4) return RHT_E_BITS;
    if (yt != RHT_F32 && yt != RHT_F16) return RHT_E_DTYPE;
    if (n == 0) return RHT_OK;
    if (!codes || !signs || !norms || !res_scale || !y) return RHT_E_NULL;
    if (!aligned(codes) || !aligned(signs) || !aligned(norms) || !aligned(res_scale) || !aligned(y))
        return RHT_E_ALIGN;

    DequantArgs a;
    std::memset(&a, 0, sizeof(a));
    a.codes = codes;
    a.signs = signs;
    a.scale = norms;
    a.res_scale = res_scale;
    a.y = y;
    a.n = n;
    std::memcpy(a.lev, book(bits - 1).lev, sizeof(a.lev));
    sign_words(seed, d, a.dsign);
    return launched(launch_dequantize(d, yt == RHT_F16, bits, kResidual, a, (hipStream_t)stream));
}

rht_status rht_score(const float *q, int32_t m, const uint8_t *codes, const float *norms, int64_t n,
                     int32_t d, int32_t bits, uint64_t seed, float *logits, void *stream) {
    if (n < 0 || m < 0 || m > 64) return RHT_E_COUNT;
    if (!pow2_dim(d)) return RHT_E_DIM;
    if (bits < 1 || bits > 4) return RHT_E_BITS;
    if (n == 0 || m == 0) return RHT_OK;
    if (!q || !codes || !norms || !logits) return RHT_E_NULL;
    if (!aligned(q) || !aligned(codes) || !aligned(norms) || !aligned(logits)) return RHT_E_ALIGN;

    ScoreArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q;
    a.m = m;
    a.codes = codes;
    a.norms = norms;
    a.logits = logits;
    a.n = n;
    a.key_mult = 1.0f / (float)d;
    std::memcpy(a.lev, book(bits).lev, sizeof(a.lev));
    sign_words(seed, d, a.dsign);
    return launched(launch_score(d, bits, false, a, (hipStream_t)stream));
}

rht_status rht_score_sign(const float *q, int32_t m, const uint8_t *bits, const float *scale, int64_t n,
                          int32_t d, uint64_t seed, float *logits, void *stream) {
    if (n < 0 || m < 0 || m > 64) return RHT_E_COUNT;
    if (!pow2_dim(d)) return RHT_E_DIM;
    if (n == 0 || m == 0) return RHT_OK;
    if (!q || !bits || !scale || !logits) return RHT_E_NULL;
    if (!aligned(q) || !aligned(bits) || !aligned(scale) || !aligned(logits)) return RHT_E_ALIGN;

    ScoreArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q;
    a.m = m;
    a.codes = bits;
    a.norms = scale;
    a.logits = logits;
    a.n = n;
    a.key_mult = 1.0f / std::sqrt((float)d);
    a.lev[0] = -1.0f;  // bit 0: the rotated coordinate was negative
    a.lev[1] = 1.0f;
    a.exact = 1;
    sign_words(seed, d, a.dsign);
    return launched(launch_score(d, 1, false, a, (hipStream_t)stream));
}

rht_status rht_residual_score(const float *q, int32_t m, const uint8_t *codes, const uint8_t *signs,
                              const float *norms, const float *res_scale, int64_t n, int32_t d, int32_t bits,
                              uint64_t seed, float *logits, void *stream) {
    if (n < 0 || m < 0 || m > 64) return RHT_E_COUNT;
    if (!pow2_dim(d)) return RHT_E_DIM;
    if (bits < 2 || bits > 4) return RHT_E_BITS;
    if (n == 0 || m == 0) return RHT_OK;
    if (!q || !codes || !signs || !norms || !res_scale || !logits) return RHT_E_NULL;
    if (!aligned(q) || !aligned(codes) || !aligned(signs) || !aligned(norms) || !aligned(res_scale) ||
        !aligned(logits))
        return RHT_E_ALIGN;

    ScoreArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q;
    a.m = m;
    a.codes = codes;
    a.norms = norms;
    a.signs = signs;
    a.res_scale = res_scale;
    a.logits = logits;
    a.n = n;
    std::memcpy(a.lev, book(bits - 1).lev, sizeof(a.lev));
    sign_words(seed, d, a.dsign);
    return launched(launch_score(d, bits - 1, true, a, (hipStream_t)stream));
}

size_t rht_attention_workspace_bytes(int64_t heads, int32_t m, int64_t n, int32_t d) {
    if (!attention_args_ok(heads, m, n) || d != 128 || heads == 0) return 0;
    return (size_t)heads * (size_t)attention_chunks(heads, n) * (size_t)m * kAttnRecord * sizeof(float);
}

namespace {

// Validation shared by the two attention entry points, up to (not including)
// the workspace: the checks and their order documented for rht_attention.
rht_status attention_check(const float *q, int32_t m, const uint8_t *k_codes, const float *k_norms,
                           const uint8_t *v_codes, const float *v_norms, int64_t heads, int64_t n, int32_t d,
                           int32_t k_bits, int32_t v_bits, const float *out) {
    if (!attention_args_ok(heads, m, n)) return RHT_E_COUNT;
    if (d != 128) return RHT_E_DIM;
    if (k_bits < 2 || k_bits > 4 || v_bits < 2 || v_bits > 4) return RHT_E_BITS;
    if (heads == 0) return RHT_OK;
    if (!q || !k_codes || !k_norms || !v_codes || !v_norms || !out) return RHT_E_NULL;
    if (!aligned(q) || !aligned(k_codes) || !aligned(k_norms) || !aligned(v_codes) || !aligned(v_norms) ||
        !aligned(out))
        return RHT_E_ALIGN;
    return RHT_OK;
}

rht_status attention_launch(const float *q, int32_t m, const uint8_t *k_codes, const float *k_norms,
                            const uint8_t *v_codes, const float *v_norms, int64_t heads, int64_t n, int32_t d,
                            int32_t k_bits, int32_t v_bits, uint64_t seed_k, uint64_t seed_v, float scale,
                            float *out, float *ws, void *stream) {
    AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q;
    a.kc = k_codes;
    a.vc = v_codes;
    a.kn = k_norms;
    a.vn = v_norms;
    a.ws = ws;
    a.out = out;
    a.heads = heads;
    a.n = n;
    a.m = m;
    a.chunks = (int)attention_chunks(heads, n);
    a.scale = scale;
    a.kbits = k_bits;
    a.vbits = v_bits;
    std::memcpy(a.lev_k, book(k_bits).lev, sizeof(a.lev_k));
    std::memcpy(a.lev_v, book(v_bits).lev, sizeof(a.lev_v));
    sign_words(seed_k, d, a.dsign_k);
    sign_words(seed_v, d, a.dsign_v);
    return launched(launch_attention(a, (hipStream_t)stream));
}

}  // namespace

rht_status rht_attention(const float *q, int32_t m, const uint8_t *k_codes, const float *k_norms,
                         const uint8_t *v_codes, const float *v_norms, int64_t heads, int64_t n,
                         int32_t d, int32_t k_bits, int32_t v_bits, uint64_t seed_k, uint64_t seed_v, float scale,
                         float *out, void *workspace, size_t workspace_bytes, void *stream) {
    const rht_status st =
        attention_check(q, m, k_codes, k_norms, v_codes, v_norms, heads, n, d, k_bits, v_bits, out);
    if (st != RHT_OK || heads == 0) return st;
    if (!workspace) return RHT_E_NULL;
    if (!aligned(workspace)) return RHT_E_ALIGN;
    if (workspace_bytes < rht_attention_workspace_bytes(heads, m, n, d)) return RHT_E_WORKSPACE;
    return attention_launch(q, m, k_codes, k_norms, v_codes, v_norms, heads, n, d, k_bits, v_bits, seed_k, seed_v,
                            scale, out, static_cast<float *>(workspace), stream);
}

rht_status rht_attention_noalloc(const float *q, int32_t m, const uint8_t *k_codes, const float *k_norms,
                                 const uint8_t *v_codes, const float *v_norms, int64_t heads, int64_t n,
                                 int32_t d, int32_t k_bits, int32_t v_bits, uint64_t seed_k, uint64_t seed_v,
                                 float scale, float *out, void *stream) {
    const rht_status st =
        attention_check(q, m, k_codes, k_norms, v_codes, v_norms, heads, n, d, k_bits, v_bits, out);
    if (st != RHT_OK || heads == 0) return st;
    if (rht_attention_workspace_bytes(heads, m, n, d) > kAttnScratchBytes) return RHT_E_WORKSPACE;
    void *ws = nullptr;
    if (attention_scratch(&ws) != hipSuccess) return RHT_E_DEVICE;
    return attention_launch(q, m, k_codes, k_norms, v_codes, v_norms, heads, n, d, k_bits, v_bits, seed_k, seed_v,
                            scale, out, static_cast<float *>(ws), stream);
}

}  // extern "C"
