/*
 * rht_oracle.c -- CPU oracle for random-rotation (randomized Hadamard)
 * vector quantization.  fp64 arithmetic throughout, single-threaded, plain C99.
 *
 * TEST INFRASTRUCTURE.  This is the reference the HIP library is checked
 * against; it is not part of the product path.  Only the test suite, the
 * package smoke check and the benchmark's CPU-baseline leg load it.  It shares
 * no code, header, table or constant generator with the HIP library.
 *
 * Source of every formula: the web page "Random-rotation quantization"
 * ("Квантование со случайным поворотом", brain.bigb.es), cited below as [RRQ]
 * with its section:
 *   [RRQ intro]      the three-step scheme (rotate by Pi, quantize every
 *                    rotated coordinate with one fixed codebook, decode with
 *                    Pi^T); the codebook is the same for every input.
 *   [RRQ why]        "Why rotation works": coordinates after a uniform
 *                    rotation have mean 0, std 1/sqrt(d), a Beta marginal;
 *                    in practice Pi is the randomized Hadamard transform,
 *                    computable in O(d log d).
 *   [RRQ DRIVE]      "History", DRIVE item: signs of the rotated coordinates
 *                    plus one scale; S = ||R(x)||_1 / d (biased, MSE-optimal)
 *                    or S = ||x||_2^2 / ||R(x)||_1 (unbiased).
 *   [RRQ EDEN]       "History", EDEN item: normalize so each rotated
 *                    coordinate is about N(0,1), quantize with the Lloyd-Max
 *                    codebook of the standard normal (1 bit: +-sqrt(2/pi);
 *                    2 bits: +-0.453, +-1.510).
 *   [RRQ TurboQuant] "History", TurboQuant item: one scale per vector and a
 *                    residual chain (b-1 biased bits + 1 unbiased bit).
 *   [RRQ decoders]   "Three decoders, one rotation": mean decoder
 *                    S * Pi^T sign(Pi x); inner-product decoder from
 *                    <Pi q, code>; MSE decoder Pi^T(centroids).
 *   [RRQ bias]       "Bias vs unbiasedness": MSE codes shrink inner products;
 *                    the residual chain (b-1 bits MSE, then a 1-bit unbiased
 *                    sign code of the residual) removes the bias.
 *   [TQ-FWHT]        page "TurboQuant and per-layer outlier-aware K",
 *                    section "TurboQuant 2026": the rotation is the fast
 *                    Walsh-Hadamard transform.
 *   [ATTN-ROT]       page "Attn-rot: TurboQuant lite in llama.cpp", opening
 *                    section: the keys and values of the attention KV cache
 *                    are rotated and quantized, attention then runs on them.
 *   [RRQ practice]   "Practical use in llama.cpp": TurboQuant codebooks as
 *                    KV-cache types for K and V.
 *
 * Readings taken where the pages are silent (each is one plain choice):
 *   - Pi = H D / sqrt(d): D = diag of seeded +-1 signs, H the Sylvester-ordered
 *     Hadamard matrix H_ij = (-1)^popcount(i & j); Pi^T = D H / sqrt(d).
 *   - seed -> signs: sign i is the top bit of the i-th SplitMix64 output
 *     (Steele, Lea, Flood 2014) started from state `seed`; bit set => -1.
 *   - normalization y = sqrt(d) (Pi x)/||x|| = (H D x)/||x||; stored scalar is
 *     ||x||_2 rounded to fp32; ||x|| = 0 gives y = 0.
 *   - codebook: Lloyd-Max for N(0,1), thresholds are midpoints, ties go up:
 *     code = #{k : y >= t_k}; the middle threshold is exactly 0.
 *   - packing: LSB-first bitstream per row, code i at bits [b*i, b*i + b).
 *   - residual scale: DRIVE's unbiased scale applied to the rotated-domain
 *     residual r, S_r = ||r||_2^2 / ||r||_1 (0 when ||r||_1 = 0).
 *   - outputs rounded to fp32 or fp16 with round-to-nearest-even.
 *   - attention: out_i = sum_j softmax_j(scale * <q_i, k~_j>) v~_j over the
 *     decoded keys k~ and values v~ (scale supplied by the caller, no mask);
 *     keys and values may use different rotation seeds.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define RHO_ABI 1

#define RHO_F32 0
#define RHO_F16 1
#define RHO_PI 3.14159265358979323846

int rho_abi(void) { return RHO_ABI; }

/* ------------------------------------------------------------------------ */
/* SplitMix64 (Steele, Lea, Flood, OOPSLA 2014): state advances by the golden
 * gamma, output is the state passed through the 64-bit finalizer.            */
uint64_t rho_splitmix64_next(uint64_t *state)
{
    uint64_t z;
    *state += 0x9E3779B97F4A7C15ULL;
    z = *state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* The random diagonal D of the randomized Hadamard transform [RRQ why]:
 * s[i] = -1 when the top bit of the i-th generator output is set.           */
void rho_signs(uint64_t seed, int d, int8_t *s)
{
    uint64_t state = seed;
    int i;
    for (i = 0; i < d; ++i) {
        uint64_t r = rho_splitmix64_next(&state);
        s[i] = (r >> 63) ? (int8_t)-1 : (int8_t)1;
    }
}

/* Unnormalized fast Walsh-Hadamard transform in Sylvester order [TQ-FWHT],
 * [RRQ why] (O(d log d)): for h = 1, 2, ..., d/2 replace every pair
 * (v[j], v[j+h]) in each block of 2h by (v[j] + v[j+h], v[j] - v[j+h]).      */
void rho_fwht(double *v, int d)
{
    int h, i, j;
    for (h = 1; h < d; h *= 2) {
        for (i = 0; i < d; i += 2 * h) {
            for (j = i; j < i + h; ++j) {
                double a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16 <-> double, written out from the format's definition.    */
double rho_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1F;
    int man = h & 0x3FF;
    double v;
    if (exp == 0)
        v = ldexp((double)man, -24); /* subnormal: man * 2^-24 */
    else if (exp == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man + 1024), exp - 25); /* (1024+man) * 2^(exp-15-10) */
    return sign ? -v : v;
}

/* Round-to-nearest-even from double; overflow to infinity. */
uint16_t rho_f64_to_f16(double v)
{
    uint16_t sign = (uint16_t)(signbit(v) ? 0x8000 : 0);
    double a = fabs(v);
    if (isnan(v)) return 0x7E00;
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00); /* halfway to 2^16 and beyond */
    if (a < ldexp(1.0, -14)) {
        double m = nearbyint(ldexp(a, 24)); /* units of 2^-24, ties to even */
        return (uint16_t)(sign | (uint16_t)m); /* m == 1024 is the smallest normal */
    } else {
        int e2;
        double f = frexp(a, &e2);      /* a = f * 2^e2, f in [0.5, 1) */
        int e = e2 - 1;                /* a in [2^e, 2^(e+1)) */
        double m = nearbyint(ldexp(f, 11)); /* a / 2^(e-10), in [1024, 2048] */
        if (m == 2048.0) { m = 1024.0; e += 1; }
        if (e + 15 >= 31) return (uint16_t)(sign | 0x7C00);
        return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)m - 1024));
    }
}

static double load_elem(const void *x, int dtype, int64_t idx)
{
    if (dtype == RHO_F16) return rho_f16_to_f64(((const uint16_t *)x)[idx]);
    return (double)((const float *)x)[idx];
}

static void store_elem(void *y, int dtype, int64_t idx, double v)
{
    if (dtype == RHO_F16)
        ((uint16_t *)y)[idx] = rho_f64_to_f16(v);
    else
        ((float *)y)[idx] = (float)v;
}

/* ------------------------------------------------------------------------ */
/* Lloyd-Max codebook for the standard normal [RRQ EDEN], [RRQ intro] (one
 * fixed codebook for every input).  Lloyd's fixed point: thresholds are the
 * midpoints of neighbouring levels, each level is the conditional mean of
 * N(0,1) on its cell, E[Z | a <= Z < b] = (phi(a) - phi(b)) / P(a <= Z < b).  */
static double std_pdf(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * RHO_PI); }

/* P(a <= Z < b) for Z ~ N(0,1), evaluated on the side that avoids cancellation. */
static double std_prob(double a, double b)
{
    const double r2 = sqrt(2.0);
    if (a >= 0.0) return 0.5 * (erfc(a / r2) - erfc(b / r2));
    if (b <= 0.0) return 0.5 * (erfc(-b / r2) - erfc(-a / r2));
    return 1.0 - 0.5 * erfc(b / r2) - 0.5 * erfc(-a / r2);
}

int rho_lloyd_max(int bits, double *levels, double *thresholds, double *mse, int *iters_out)
{
    int K, k, it;
    double c[16], t[17];
    if (bits < 1 || bits > 4) return -1;
    K = 1 << bits;
    for (k = 0; k < K; ++k) c[k] = -3.0 + 6.0 * (k + 0.5) / K; /* uniform start */
    for (it = 0; it < 1000000; ++it) {
        double delta = 0.0;
        t[0] = -INFINITY;
        t[K] = INFINITY;
        for (k = 1; k < K; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
        for (k = 0; k < K; ++k) {
            double pa = isinf(t[k]) ? 0.0 : std_pdf(t[k]);
            double pb = isinf(t[k + 1]) ? 0.0 : std_pdf(t[k + 1]);
            double cn = (pa - pb) / std_prob(t[k], t[k + 1]);
            double dd = fabs(cn - c[k]);
            if (dd > delta) delta = dd;
            c[k] = cn;
        }
        if (delta < 1e-14) break;
    }
    /* the N(0,1) density is even, so the fixed point is antisymmetric */
    for (k = 0; k < K / 2; ++k) {
        double m = 0.5 * (c[K - 1 - k] - c[k]);
        c[k] = -m;
        c[K - 1 - k] = m;
    }
    for (k = 1; k < K; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    t[K / 2] = 0.0;
    t[0] = -INFINITY;
    t[K] = INFINITY;
    if (mse) {
        /* D_b = E[(Z - c(Z))^2] = 1 - sum_k p_k c_k^2 when c_k are cell means */
        double s = 0.0;
        for (k = 0; k < K; ++k) s += std_prob(t[k], t[k + 1]) * c[k] * c[k];
        *mse = 1.0 - s;
    }
    for (k = 0; k < K; ++k) levels[k] = c[k];
    for (k = 1; k < K; ++k) thresholds[k - 1] = t[k];
    if (iters_out) *iters_out = it;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Lloyd-Max codebook for the exact finite-d marginal [RRQ why]: a coordinate
 * t of a uniformly rotated unit vector in R^d has density proportional to
 * (1 - t^2)^((d-3)/2) on [-1, 1] (a Beta law), so y = sqrt(d) t (variance 1)
 * has density proportional to (1 - y^2/d)^((d-3)/2) on [-sqrt(d), sqrt(d)].
 * With y = sqrt(d) sin(theta) a cell [a, b) has mass proportional to the
 * integral of cos(theta)^(d-2) over [asin(a/sqrt d), asin(b/sqrt d)) and first
 * moment sqrt(d) * integral of sin(theta) cos(theta)^(d-2); both integrands
 * are smooth, so composite Simpson's rule gives them to rounding.  Lloyd's
 * fixed point as for N(0,1), started from the N(0,1) codebook.  d >= 2.     */
static double beta_cell_integral(double ta, double tb, int d, int moment)
{
    /* |y| > 12 carries less than exp(-72) of the mass (the tails are lighter
     * than the normal law's): clip there so the points sit where the mass is */
    const int N = 4000; /* Simpson intervals per cell (even) */
    const double tmax = asin(fmin(1.0, 12.0 / sqrt((double)d)));
    double h, acc = 0.0;
    int i;
    ta = fmax(ta, -tmax);
    tb = fmin(tb, tmax);
    if (tb <= ta) return 0.0;
    h = (tb - ta) / N;
    for (i = 0; i <= N; ++i) {
        double th = ta + h * i;
        double f = pow(cos(th), (double)(d - 2)) * (moment ? sin(th) : 1.0);
        acc += f * (i == 0 || i == N ? 1.0 : (i % 2 ? 4.0 : 2.0));
    }
    return acc * h / 3.0;
}

int rho_lloyd_max_beta(int bits, int d, double *levels, double *thresholds, double *mse, int *iters_out)
{
    double c[16], t[17], rd = sqrt((double)d), total;
    int K, k, it;
    if (bits < 1 || bits > 4 || d < 2) return -1;
    K = 1 << bits;
    rho_lloyd_max(bits, c, t + 1, NULL, NULL);
    /* start inside the support [-sqrt(d), sqrt(d)] */
    if (c[K - 1] >= 0.9 * rd)
        for (k = 0; k < K; ++k) c[k] *= 0.9 * rd / c[K - 1];
    total = beta_cell_integral(-RHO_PI / 2, RHO_PI / 2, d, 0);
    for (it = 0; it < 100000; ++it) {
        double delta = 0.0;
        t[0] = -RHO_PI / 2;
        t[K] = RHO_PI / 2;
        for (k = 1; k < K; ++k) {
            double m = 0.5 * (c[k - 1] + c[k]);
            if (m < -rd) m = -rd;
            if (m > rd) m = rd;
            t[k] = asin(m / rd);
        }
        for (k = 0; k < K; ++k) {
            double z = beta_cell_integral(t[k], t[k + 1], d, 0);
            double m1 = rd * beta_cell_integral(t[k], t[k + 1], d, 1);
            double nc = z > 0.0 ? m1 / z : c[k];
            if (fabs(nc - c[k]) > delta) delta = fabs(nc - c[k]);
            c[k] = nc;
        }
        if (delta < 1e-14) break;
    }
    /* symmetrize; the middle threshold is exactly 0 */
    for (k = 0; k < K / 2; ++k) {
        double a = 0.5 * (c[K - 1 - k] - c[k]);
        c[k] = -a;
        c[K - 1 - k] = a;
    }
    for (k = 0; k < K; ++k) levels[k] = c[k];
    for (k = 1; k < K; ++k) thresholds[k - 1] = k == K / 2 ? 0.0 : 0.5 * (c[k - 1] + c[k]);
    if (mse) {
        /* E[(Y - c(Y))^2] = E[Y^2] - sum_k P_k c_k^2 = 1 - sum_k P_k c_k^2 (centroid rule) */
        double acc = 0.0;
        for (k = 0; k < K; ++k) {
            double lo = k == 0 ? -RHO_PI / 2 : asin(fmax(-1.0, fmin(1.0, thresholds[k - 1] / rd)));
            double hi = k == K - 1 ? RHO_PI / 2 : asin(fmax(-1.0, fmin(1.0, thresholds[k] / rd)));
            acc += beta_cell_integral(lo, hi, d, 0) / total * c[k] * c[k];
        }
        *mse = 1.0 - acc;
    }
    if (iters_out) *iters_out = it;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* bit packing: LSB-first bitstream, field i at bits [w*i, w*i + w)          */
static void put_field(uint8_t *row, int i, int w, unsigned v)
{
    int j;
    for (j = 0; j < w; ++j) {
        int64_t bit = (int64_t)w * i + j;
        if ((v >> j) & 1u) row[bit >> 3] |= (uint8_t)(1u << (bit & 7));
    }
}

static unsigned get_field(const uint8_t *row, int i, int w)
{
    unsigned v = 0;
    int j;
    for (j = 0; j < w; ++j) {
        int64_t bit = (int64_t)w * i + j;
        v |= (unsigned)((row[bit >> 3] >> (bit & 7)) & 1u) << j;
    }
    return v;
}

static int valid_dim(int d) { return d >= 1 && d <= (1 << 16) && (d & (d - 1)) == 0; }

/* h = H D x for one row, plus ||x||^2.  */
static void rotate_row(const void *x, int dtype, int64_t row, int d, const int8_t *s,
                       double *h, double *sumsq)
{
    int i;
    double ss = 0.0;
    for (i = 0; i < d; ++i) {
        double v = load_elem(x, dtype, row * d + i);
        ss += v * v;
        h[i] = s[i] * v;
    }
    rho_fwht(h, d);
    *sumsq = ss;
}

/* EDEN/TurboQuant MSE encoder [RRQ intro], [RRQ EDEN], [RRQ TurboQuant]:
 * y = H D x / ||x|| (= sqrt(d) * Pi x / ||x||, each coordinate ~ N(0,1)),
 * code_i = nearest Lloyd-Max level = #{k : y_i >= t_k}, norm = ||x||_2.
 * y_out (optional, [n][d]) receives y in fp64 for near-threshold accounting.  */
int rho_quantize(const void *x, int dtype, int64_t n, int d, int bits, uint64_t seed,
                 uint8_t *codes, float *norms, double *y_out)
{
    double lv[16], th[15];
    int8_t *s;
    double *h;
    int64_t r;
    int i, k, K, row_bytes;
    if (!valid_dim(d) || bits < 1 || bits > 4 || n < 0) return -1;
    if ((int64_t)bits * d % 8) return -1;
    K = 1 << bits;
    row_bytes = bits * d / 8;
    rho_lloyd_max(bits, lv, th, NULL, NULL);
    s = (int8_t *)malloc((size_t)d);
    h = (double *)malloc(sizeof(double) * (size_t)d);
    rho_signs(seed, d, s);
    for (r = 0; r < n; ++r) {
        double ss, nrm;
        uint8_t *crow = codes + r * row_bytes;
        rotate_row(x, dtype, r, d, s, h, &ss);
        nrm = sqrt(ss);
        memset(crow, 0, (size_t)row_bytes);
        for (i = 0; i < d; ++i) {
            double y = nrm > 0.0 ? h[i] / nrm : 0.0;
            unsigned code = 0;
            for (k = 0; k < K - 1; ++k)
                if (y >= th[k]) ++code;
            put_field(crow, i, bits, code);
            if (y_out) y_out[r * d + i] = y;
        }
        norms[r] = (float)nrm;
    }
    free(h);
    free(s);
    return 0;
}

/* EDEN-style unbiased scale for the MSE codes [RRQ EDEN], [RRQ bias]
 * (reading: DRIVE's unbiased scale carried over to the Lloyd-Max code): the
 * codes are the MSE encoder's; the stored scalar is the S that makes the
 * decoder x^ = D H (c S / d) satisfy <x^, x> = ||x||^2,
 *   S = d ||x||^2 / <c[code], H D x>   (0 when that inner product is 0).
 * The MSE decoder (rho_dequantize) decodes it unchanged.                     */
int rho_quantize_eden(const void *x, int dtype, int64_t n, int d, int bits, uint64_t seed,
                      uint8_t *codes, float *scale)
{
    double lv[16], th[15];
    int8_t *s;
    double *h;
    int64_t r;
    int i, k, K, row_bytes;
    if (!valid_dim(d) || bits < 1 || bits > 4 || n < 0) return -1;
    if ((int64_t)bits * d % 8) return -1;
    K = 1 << bits;
    row_bytes = bits * d / 8;
    rho_lloyd_max(bits, lv, th, NULL, NULL);
    s = (int8_t *)malloc((size_t)d);
    h = (double *)malloc(sizeof(double) * (size_t)d);
    rho_signs(seed, d, s);
    for (r = 0; r < n; ++r) {
        double ss, nrm, ch = 0.0;
        uint8_t *crow = codes + r * row_bytes;
        rotate_row(x, dtype, r, d, s, h, &ss);
        nrm = sqrt(ss);
        memset(crow, 0, (size_t)row_bytes);
        for (i = 0; i < d; ++i) {
            double y = nrm > 0.0 ? h[i] / nrm : 0.0;
            unsigned code = 0;
            for (k = 0; k < K - 1; ++k)
                if (y >= th[k]) ++code;
            put_field(crow, i, bits, code);
            ch += lv[code] * h[i];
        }
        scale[r] = (float)(ch != 0.0 ? d * ss / ch : 0.0);
    }
    free(h);
    free(s);
    return 0;
}

/* MSE decoder [RRQ decoders], [RRQ intro] step 3: x~ = Pi^T (c * ||x|| / sqrt(d))
 * = D H (c * ||x|| / d), from the stored bytes only.                         */
int rho_dequantize(const uint8_t *codes, const float *norms, int64_t n, int d, int bits,
                   uint64_t seed, void *out, int out_dtype)
{
    double lv[16], th[15];
    int8_t *s;
    double *z;
    int64_t r;
    int i, row_bytes;
    if (!valid_dim(d) || bits < 1 || bits > 4 || n < 0) return -1;
    if ((int64_t)bits * d % 8) return -1;
    row_bytes = bits * d / 8;
    rho_lloyd_max(bits, lv, th, NULL, NULL);
    s = (int8_t *)malloc((size_t)d);
    z = (double *)malloc(sizeof(double) * (size_t)d);
    rho_signs(seed, d, s);
    for (r = 0; r < n; ++r) {
        const uint8_t *crow = codes + r * row_bytes;
        double scale = (double)norms[r] / d;
        for (i = 0; i < d; ++i) z[i] = lv[get_field(crow, i, bits)] * scale;
        rho_fwht(z, d);
        for (i = 0; i < d; ++i) store_elem(out, out_dtype, r * d + i, s[i] * z[i]);
    }
    free(z);
    free(s);
    return 0;
}

/* The MSE encoder and decoder with a codebook given by the caller (levels
 * ascending, thresholds[k] between levels k and k+1): used for the exact
 * finite-d codebook; identical to rho_quantize / rho_dequantize otherwise.   */
int rho_quantize_cb(const void *x, int dtype, int64_t n, int d, int bits, uint64_t seed,
                    const double *levels, const double *thresholds, uint8_t *codes, float *norms,
                    double *y_out)
{
    int8_t *s;
    double *h;
    int64_t r;
    int i, k, K, row_bytes;
    (void)levels;
    if (!valid_dim(d) || bits < 1 || bits > 4 || n < 0) return -1;
    if ((int64_t)bits * d % 8) return -1;
    K = 1 << bits;
    row_bytes = bits * d / 8;
    s = (int8_t *)malloc((size_t)d);
    h = (double *)malloc(sizeof(double) * (size_t)d);
    rho_signs(seed, d, s);
    for (r = 0; r < n; ++r) {
        double ss, nrm;
        uint8_t *crow = codes + r * row_bytes;
        rotate_row(x, dtype, r, d, s, h, &ss);
        nrm = sqrt(ss);
        memset(crow, 0, (size_t)row_bytes);
        for (i = 0; i < d; ++i) {
            double y = nrm > 0.0 ? h[i] / nrm : 0.0;
            unsigned code = 0;
            for (k = 0; k < K - 1; ++k)
                if (y >= thresholds[k]) ++code;
            put_field(crow, i, bits, code);
            if (y_out) y_out[r * d + i] = y;
        }
        norms[r] = (float)nrm;
    }
    free(h);
    free(s);
    return 0;
}

int rho_dequantize_cb(const uint8_t *codes, const float *norms, int64_t n, int d, int bits, uint64_t seed,
                      const double *levels, void *out, int out_dtype)
{
    int8_t *s;
    double *z;
    int64_t r;
    int i, row_bytes;
    if (!valid_dim(d) || bits < 1 || bits > 4 || n < 0) return -1;
    if ((int64_t)bits * d % 8) return -1;
    row_bytes = bits * d / 8;
    s = (int8_t *)malloc((size_t)d);
    z = (double *)malloc(sizeof(double) * (size_t)d);
    rho_signs(seed, d, s);
    for (r = 0; r < n; ++r) {
        const uint8_t *crow = codes + r * row_bytes;
        double scale = (double)norms[r] / d;
        for (i = 0; i < d; ++i) z[i] = levels[get_field(crow, i, bits)] * scale;
        rho_fwht(z, d);
        for (i = 0; i < d; ++i) store_elem(out, out_dtype, r * d + i, s[i] * z[i]);
    }
    free(z);
    free(s);
    return 0;
}

/* DRIVE 1-bit encoder [RRQ DRIVE]: R(x) = Pi x = H D x / sqrt(d);
 * bit_i = [R(x)_i >= 0]; S = ||R(x)||_1 / d (biased) or ||x||^2 / ||R(x)||_1
 * (unbiased, 0 when ||R(x)||_1 = 0).  y_out: H D x / ||x|| as in rho_quantize. */
int rho_sign_quantize(const void *x, int dtype, int64_t n, int d, int unbiased, uint64_t seed,
                      uint8_t *bits, float *scale, double *y_out)
{
    int8_t *s;
    double *h;
    int64_t r;
    int i, row_bytes;
    double rd = sqrt((double)d);
    if (!valid_dim(d) || d < 8 || n < 0) return -1;
    row_bytes = d / 8;
    s = (int8_t *)malloc((size_t)d);
    h = (double *)malloc(sizeof(double) * (size_t)d);
    rho_signs(seed, d, s);
    for (r = 0; r < n; ++r) {
        double ss, l1 = 0.0, nrm, S;
        uint8_t *brow = bits + r * row_bytes;
        rotate_row(x, dtype, r, d, s, h, &ss);
        nrm = sqrt(ss);
        memset(brow, 0, (size_t)row_bytes);
        for (i = 0; i < d; ++i) {
            double rx = h[i] / rd; /* R(x)_i */
            l1 += fabs(rx);
            put_field(brow, i, 1, h[i] >= 0.0 ? 1u : 0u);
            if (y_out) y_out[r * d + i] = nrm > 0.0 ? h[i] / nrm : 0.0;
        }
        if (unbiased)
            S = l1 > 0.0 ? ss / l1 : 0.0;
        else
            S = l1 / d;
        scale[r] = (float)S;
    }
    free(h);
    free(s);
    return 0;
}

/* DRIVE mean decoder [RRQ decoders]: x^ = S * Pi^T sign = S * D H sigma / sqrt(d),
 * sigma_i = +1 for a set bit, -1 otherwise.                                  */
int rho_sign_dequantize(const uint8_t *bits, const float *scale, int64_t n, int d, uint64_t seed,
                        void *out, int out_dtype)
{
    int8_t *s;
    double *z;
    int64_t r;
    int i, row_bytes;
    double rd = sqrt((double)d);
    if (!valid_dim(d) || d < 8 || n < 0) return -1;
    row_bytes = d / 8;
    s = (int8_t *)malloc((size_t)d);
    z = (double *)malloc(sizeof(double) * (size_t)d);
    rho_signs(seed, d, s);
    for (r = 0; r < n; ++r) {
        const uint8_t *brow = bits + r * row_bytes;
        double S = (double)scale[r];
        for (i = 0; i < d; ++i) z[i] = get_field(brow, i, 1) ? 1.0 : -1.0;
        rho_fwht(z, d);
        for (i = 0; i < d; ++i) store_elem(out, out_dtype, r * d + i, S * s[i] * z[i] / rd);
    }
    free(z);
    free(s);
    return 0;
}

/* Residual chain [RRQ TurboQuant], [RRQ bias]: stage 1 is the (b-1)-bit MSE
 * encoder; the rotated-domain residual r = Pi (x - x~) = (h - ||x|| c) / sqrt(d)
 * gets a 1-bit sign code, sbit_i = [r_i >= 0], with DRIVE's unbiased scale
 * S_r = ||r||_2^2 / ||r||_1.  When forced_codes is given, those stage-1 codes
 * are used instead of the oracle's own (downstream parity on identical codes). */
int rho_residual_quantize(const void *x, int dtype, int64_t n, int d, int bits, uint64_t seed,
                          const uint8_t *forced_codes, uint8_t *codes, uint8_t *signs,
                          float *norms, float *res_scale, double *y_out)
{
    double lv[16], th[15];
    int8_t *s;
    double *h;
    int64_t r;
    int i, k, b1 = bits - 1, K1, crow_bytes, srow_bytes;
    double rd = sqrt((double)d);
    if (!valid_dim(d) || d < 8 || bits < 2 || bits > 5 || n < 0) return -1;
    if ((int64_t)b1 * d % 8) return -1;
    K1 = 1 << b1;
    crow_bytes = b1 * d / 8;
    srow_bytes = d / 8;
    rho_lloyd_max(b1, lv, th, NULL, NULL);
    s = (int8_t *)malloc((size_t)d);
    h = (double *)malloc(sizeof(double) * (size_t)d);
    rho_signs(seed, d, s);
    for (r = 0; r < n; ++r) {
        double ss, nrm, r2 = 0.0, r1 = 0.0;
        uint8_t *crow = codes + r * crow_bytes;
        uint8_t *srow = signs + r * srow_bytes;
        rotate_row(x, dtype, r, d, s, h, &ss);
        nrm = sqrt(ss);
        memset(srow, 0, (size_t)srow_bytes);
        if (!forced_codes) memset(crow, 0, (size_t)crow_bytes);
        for (i = 0; i < d; ++i) {
            double y = nrm > 0.0 ? h[i] / nrm : 0.0;
            unsigned code;
            double ri;
            if (forced_codes) {
                code = get_field(forced_codes + r * crow_bytes, i, b1);
            } else {
                code = 0;
                for (k = 0; k < K1 - 1; ++k)
                    if (y >= th[k]) ++code;
                put_field(crow, i, b1, code);
            }
            ri = (h[i] - nrm * lv[code]) / rd;
            r2 += ri * ri;
            r1 += fabs(ri);
            put_field(srow, i, 1, ri >= 0.0 ? 1u : 0u);
            if (y_out) y_out[r * d + i] = y;
        }
        if (forced_codes) memmove(crow, forced_codes + r * crow_bytes, (size_t)crow_bytes);
        norms[r] = (float)nrm;
        res_scale[r] = (float)(r1 > 0.0 ? r2 / r1 : 0.0);
    }
    free(h);
    free(s);
    return 0;
}

/* Residual-chain decoder: x^ = Pi^T (c ||x|| / sqrt(d) + S_r sigma)
 * = D H (c ||x|| / d + S_r sigma / sqrt(d)).                                 */
int rho_residual_dequantize(const uint8_t *codes, const uint8_t *signs, const float *norms,
                            const float *res_scale, int64_t n, int d, int bits, uint64_t seed,
                            void *out, int out_dtype)
{
    double lv[16], th[15];
    int8_t *s;
    double *z;
    int64_t r;
    int i, b1 = bits - 1, crow_bytes, srow_bytes;
    double rd = sqrt((double)d);
    if (!valid_dim(d) || d < 8 || bits < 2 || bits > 5 || n < 0) return -1;
    if ((int64_t)b1 * d % 8) return -1;
    crow_bytes = b1 * d / 8;
    srow_bytes = d / 8;
    rho_lloyd_max(b1, lv, th, NULL, NULL);
    s = (int8_t *)malloc((size_t)d);
    z = (double *)malloc(sizeof(double) * (size_t)d);
    rho_signs(seed, d, s);
    for (r = 0; r < n; ++r) {
        const uint8_t *crow = codes + r * crow_bytes;
        const uint8_t *srow = signs + r * srow_bytes;
        double a = (double)norms[r] / d, sr = (double)res_scale[r] / rd;
        for (i = 0; i < d; ++i)
            z[i] = lv[get_field(crow, i, b1)] * a + (get_field(srow, i, 1) ? sr : -sr);
        rho_fwht(z, d);
        for (i = 0; i < d; ++i) store_elem(out, out_dtype, r * d + i, s[i] * z[i]);
    }
    free(z);
    free(s);
    return 0;
}

/* Scoring on the codes in the rotated domain [RRQ decoders] (inner-product
 * decoder idea): <q, x~> = <q, D H c ||x|| / d> = (||x|| / d) <H D q, c>.
 * q~ = H D q is formed once per query; logits[j][k] = (||x_k|| / d) *
 * sum_i q~_{j,i} c[code_{k,i}], rounded to fp32.                             */
int rho_score(const float *q, int m, const uint8_t *codes, const float *norms, int64_t n, int d,
              int bits, uint64_t seed, float *logits)
{
    double lv[16], th[15];
    int8_t *s;
    double *qt;
    int64_t k;
    int i, j, row_bytes;
    if (!valid_dim(d) || bits < 1 || bits > 4 || n < 0 || m < 0) return -1;
    if ((int64_t)bits * d % 8) return -1;
    row_bytes = bits * d / 8;
    rho_lloyd_max(bits, lv, th, NULL, NULL);
    s = (int8_t *)malloc((size_t)d);
    qt = (double *)malloc(sizeof(double) * (size_t)d * (size_t)(m > 0 ? m : 1));
    rho_signs(seed, d, s);
    for (j = 0; j < m; ++j) {
        for (i = 0; i < d; ++i) qt[(int64_t)j * d + i] = s[i] * (double)q[(int64_t)j * d + i];
        rho_fwht(qt + (int64_t)j * d, d);
    }
    for (k = 0; k < n; ++k) {
        const uint8_t *crow = codes + k * row_bytes;
        double a = (double)norms[k] / d;
        for (j = 0; j < m; ++j) {
            double acc = 0.0;
            for (i = 0; i < d; ++i) acc += qt[(int64_t)j * d + i] * lv[get_field(crow, i, bits)];
            logits[(int64_t)j * n + k] = (float)(a * acc);
        }
    }
    free(qt);
    free(s);
    return 0;
}

/* The plain definition scoring must reach: logits = Q * dequant(K)^T, with the
 * dequantized keys kept in fp64 (no output rounding), fp64 result.           */
int rho_score_dense(const float *q, int m, const uint8_t *codes, const float *norms, int64_t n,
                    int d, int bits, uint64_t seed, double *logits)
{
    double lv[16], th[15];
    int8_t *s;
    double *z;
    int64_t k;
    int i, j, row_bytes;
    if (!valid_dim(d) || bits < 1 || bits > 4 || n < 0 || m < 0) return -1;
    if ((int64_t)bits * d % 8) return -1;
    row_bytes = bits * d / 8;
    rho_lloyd_max(bits, lv, th, NULL, NULL);
    s = (int8_t *)malloc((size_t)d);
    z = (double *)malloc(sizeof(double) * (size_t)d);
    rho_signs(seed, d, s);
    for (k = 0; k < n; ++k) {
        const uint8_t *crow = codes + k * row_bytes;
        double a = (double)norms[k] / d;
        for (i = 0; i < d; ++i) z[i] = lv[get_field(crow, i, bits)] * a;
        rho_fwht(z, d);
        for (i = 0; i < d; ++i) z[i] *= s[i];
        for (j = 0; j < m; ++j) {
            double acc = 0.0;
            for (i = 0; i < d; ++i) acc += (double)q[(int64_t)j * d + i] * z[i];
            logits[(int64_t)j * n + k] = acc;
        }
    }
    free(z);
    free(s);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention over coded keys and values [ATTN-ROT], [RRQ practice],
 * [RRQ decoders] (MSE decoder for the KV cache).  The plain definition:
 * decode every key and value in fp64 (x~ = D H c ||x|| / d, no rounding),
 * logits s_j = scale <q, k~_j>, p = softmax(s), out = sum_j p_j v~_j.
 * Keys and values may use different code widths (page "Random-rotation
 * quantization", "Practical use in llama.cpp": the K and V caches take their
 * own code types, e.g. 4-bit keys with 3-bit values); each is decoded with the
 * Lloyd-Max codebook of its own width.
 * q [heads][m][d] fp32, codes [heads][n][kbits d / 8] and [heads][n][vbits d / 8],
 * norms [heads][n], out [heads][m][d] fp64.  n >= 1.                        */
static void decode_row_f64(const uint8_t *crow, double norm, int d, int bits, const double *lv,
                           const int8_t *s, double *out)
{
    int i;
    for (i = 0; i < d; ++i) out[i] = lv[get_field(crow, i, bits)] * (norm / d);
    rho_fwht(out, d);
    for (i = 0; i < d; ++i) out[i] *= s[i];
}

int rho_attention(const float *q, int m, const uint8_t *kc, const float *kn, const uint8_t *vc,
                  const float *vn, int64_t heads, int64_t n, int d, int kbits, int vbits, uint64_t seed_k,
                  uint64_t seed_v, double scale, double *out)
{
    double lk[16], lvv[16], th[15];
    int8_t *sk, *sv;
    double *kd, *vd, *logit;
    int64_t b, j;
    int i, t, krow, vrow;
    if (!valid_dim(d) || kbits < 1 || kbits > 4 || vbits < 1 || vbits > 4 || n < 1 || m < 0 || heads < 0)
        return -1;
    if ((int64_t)kbits * d % 8 || (int64_t)vbits * d % 8) return -1;
    krow = kbits * d / 8;
    vrow = vbits * d / 8;
    rho_lloyd_max(kbits, lk, th, NULL, NULL);
    rho_lloyd_max(vbits, lvv, th, NULL, NULL);
    sk = (int8_t *)malloc((size_t)d);
    sv = (int8_t *)malloc((size_t)d);
    kd = (double *)malloc(sizeof(double) * (size_t)(n * d));
    vd = (double *)malloc(sizeof(double) * (size_t)(n * d));
    logit = (double *)malloc(sizeof(double) * (size_t)n);
    rho_signs(seed_k, d, sk);
    rho_signs(seed_v, d, sv);
    for (b = 0; b < heads; ++b) {
        for (j = 0; j < n; ++j) {
            decode_row_f64(kc + (b * n + j) * krow, kn[b * n + j], d, kbits, lk, sk, kd + j * d);
            decode_row_f64(vc + (b * n + j) * vrow, vn[b * n + j], d, vbits, lvv, sv, vd + j * d);
        }
        for (i = 0; i < m; ++i) {
            const float *qi = q + (b * m + i) * d;
            double *oi = out + (b * m + i) * d;
            double mx = -INFINITY, sum = 0.0;
            for (j = 0; j < n; ++j) {
                double acc = 0.0;
                for (t = 0; t < d; ++t) acc += (double)qi[t] * kd[j * d + t];
                logit[j] = scale * acc;
                if (logit[j] > mx) mx = logit[j];
            }
            for (t = 0; t < d; ++t) oi[t] = 0.0;
            for (j = 0; j < n; ++j) {
                double p = exp(logit[j] - mx);
                sum += p;
                for (t = 0; t < d; ++t) oi[t] += p * vd[j * d + t];
            }
            for (t = 0; t < d; ++t) oi[t] /= sum;
        }
    }
    free(logit);
    free(vd);
    free(kd);
    free(sv);
    free(sk);
    return 0;
}

/* The same attention computed in the rotated domains, as the decoders allow
 * [RRQ decoders]: the logits come from the codes, s_j = scale (||k_j|| / d)
 * <H D_k q, c[code_kj]>; the value sum stays rotated, z = sum_j p_j
 * (||v_j|| / d) c[code_vj], and one inverse transform per query gives
 * out = D_v H z (Pi_v^T is linear, so it moves out of the sum).             */
int rho_attention_rotated(const float *q, int m, const uint8_t *kc, const float *kn,
                          const uint8_t *vc, const float *vn, int64_t heads, int64_t n, int d,
                          int kbits, int vbits, uint64_t seed_k, uint64_t seed_v, double scale, double *out)
{
    double lk[16], lvv[16], th[15];
    int8_t *sk, *sv;
    double *qt, *logit;
    int64_t b, j;
    int i, t, krow, vrow;
    if (!valid_dim(d) || kbits < 1 || kbits > 4 || vbits < 1 || vbits > 4 || n < 1 || m < 0 || heads < 0)
        return -1;
    if ((int64_t)kbits * d % 8 || (int64_t)vbits * d % 8) return -1;
    krow = kbits * d / 8;
    vrow = vbits * d / 8;
    rho_lloyd_max(kbits, lk, th, NULL, NULL);
    rho_lloyd_max(vbits, lvv, th, NULL, NULL);
    sk = (int8_t *)malloc((size_t)d);
    sv = (int8_t *)malloc((size_t)d);
    qt = (double *)malloc(sizeof(double) * (size_t)d);
    logit = (double *)malloc(sizeof(double) * (size_t)n);
    rho_signs(seed_k, d, sk);
    rho_signs(seed_v, d, sv);
    for (b = 0; b < heads; ++b) {
        for (i = 0; i < m; ++i) {
            const float *qi = q + (b * m + i) * d;
            double *z = out + (b * m + i) * d;
            double mx = -INFINITY, sum = 0.0;
            for (t = 0; t < d; ++t) qt[t] = sk[t] * (double)qi[t];
            rho_fwht(qt, d);
            for (j = 0; j < n; ++j) {
                const uint8_t *crow = kc + (b * n + j) * krow;
                double acc = 0.0;
                for (t = 0; t < d; ++t) acc += qt[t] * lk[get_field(crow, t, kbits)];
                logit[j] = scale * ((double)kn[b * n + j] / d) * acc;
                if (logit[j] > mx) mx = logit[j];
            }
            for (t = 0; t < d; ++t) z[t] = 0.0;
            for (j = 0; j < n; ++j) {
                const uint8_t *crow = vc + (b * n + j) * vrow;
                double p = exp(logit[j] - mx), w;
                sum += p;
                w = p * ((double)vn[b * n + j] / d);
                for (t = 0; t < d; ++t) z[t] += w * lvv[get_field(crow, t, vbits)];
            }
            for (t = 0; t < d; ++t) z[t] /= sum;
            rho_fwht(z, d);
            for (t = 0; t < d; ++t) z[t] *= sv[t];
        }
    }
    free(logit);
    free(qt);
    free(sv);
    free(sk);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Inner products with sign-coded and residual-coded keys [RRQ decoders]
 * (inner-product decoder: <q, x> from <Pi q, sign(Pi x)> with a normalizing
 * scalar), [RRQ bias] (the residual chain restores unbiased inner products).
 * Both are <q, x^> for the vector x^ the matching decoder returns; since
 * Pi^T = D H / sqrt(d) and H is symmetric, <q, D H z> = <H D q, z>, so the
 * query is rotated once and the codes are used as they are:
 *   sign codes:  x^ = S D H sigma / sqrt(d)  ->  (S / sqrt(d)) <H D q, sigma>
 *   residual:    x^ = D H (||x|| c / d + S_r sigma / sqrt(d))
 *                ->  (||x|| / d) <H D q, c> + (S_r / sqrt(d)) <H D q, sigma>
 * sigma_i = +1 for a set bit, -1 otherwise.  Logits [m][n], rounded to fp32. */
static double *rotate_queries(const float *q, int m, int d, const int8_t *s)
{
    double *qt = (double *)malloc(sizeof(double) * (size_t)d * (size_t)(m > 0 ? m : 1));
    int i, j;
    for (j = 0; j < m; ++j) {
        for (i = 0; i < d; ++i) qt[(int64_t)j * d + i] = s[i] * (double)q[(int64_t)j * d + i];
        rho_fwht(qt + (int64_t)j * d, d);
    }
    return qt;
}

int rho_score_sign(const float *q, int m, const uint8_t *bits, const float *scale, int64_t n, int d,
                   uint64_t seed, float *logits)
{
    int8_t *s;
    double *qt;
    int64_t k;
    int i, j;
    double rd = sqrt((double)d);
    if (!valid_dim(d) || d < 8 || n < 0 || m < 0) return -1;
    s = (int8_t *)malloc((size_t)d);
    rho_signs(seed, d, s);
    qt = rotate_queries(q, m, d, s);
    for (k = 0; k < n; ++k) {
        const uint8_t *brow = bits + k * (d / 8);
        for (j = 0; j < m; ++j) {
            double acc = 0.0;
            for (i = 0; i < d; ++i)
                acc += qt[(int64_t)j * d + i] * (get_field(brow, i, 1) ? 1.0 : -1.0);
            logits[(int64_t)j * n + k] = (float)((double)scale[k] / rd * acc);
        }
    }
    free(qt);
    free(s);
    return 0;
}

int rho_score_residual(const float *q, int m, const uint8_t *codes, const uint8_t *signs,
                       const float *norms, const float *res_scale, int64_t n, int d, int bits,
                       uint64_t seed, float *logits)
{
    double lv[16], th[15];
    int8_t *s;
    double *qt;
    int64_t k;
    int i, j, b1 = bits - 1;
    double rd = sqrt((double)d);
    if (!valid_dim(d) || d < 8 || bits < 2 || bits > 5 || n < 0 || m < 0) return -1;
    if ((int64_t)b1 * d % 8) return -1;
    rho_lloyd_max(b1, lv, th, NULL, NULL);
    s = (int8_t *)malloc((size_t)d);
    rho_signs(seed, d, s);
    qt = rotate_queries(q, m, d, s);
    for (k = 0; k < n; ++k) {
        const uint8_t *crow = codes + k * (b1 * d / 8);
        const uint8_t *srow = signs + k * (d / 8);
        for (j = 0; j < m; ++j) {
            double ac = 0.0, as = 0.0;
            for (i = 0; i < d; ++i) {
                ac += qt[(int64_t)j * d + i] * lv[get_field(crow, i, b1)];
                as += qt[(int64_t)j * d + i] * (get_field(srow, i, 1) ? 1.0 : -1.0);
            }
            logits[(int64_t)j * n + k] =
                (float)((double)norms[k] / d * ac + (double)res_scale[k] / rd * as);
        }
    }
    free(qt);
    free(s);
    return 0;
}

/* The plain definitions: decode every key in fp64 with its decoder, then
 * logits = Q * x^T in fp64 (no rounding of x^ or of the result).            */
int rho_score_sign_dense(const float *q, int m, const uint8_t *bits, const float *scale, int64_t n,
                         int d, uint64_t seed, double *logits)
{
    int8_t *s;
    double *z;
    int64_t k;
    int i, j;
    double rd = sqrt((double)d);
    if (!valid_dim(d) || d < 8 || n < 0 || m < 0) return -1;
    s = (int8_t *)malloc((size_t)d);
    z = (double *)malloc(sizeof(double) * (size_t)d);
    rho_signs(seed, d, s);
    for (k = 0; k < n; ++k) {
        const uint8_t *brow = bits + k * (d / 8);
        for (i = 0; i < d; ++i) z[i] = get_field(brow, i, 1) ? 1.0 : -1.0;
        rho_fwht(z, d);
        for (i = 0; i < d; ++i) z[i] *= (double)scale[k] * s[i] / rd;
        for (j = 0; j < m; ++j) {
            double acc = 0.0;
            for (i = 0; i < d; ++i) acc += (double)q[(int64_t)j * d + i] * z[i];
            logits[(int64_t)j * n + k] = acc;
        }
    }
    free(z);
    free(s);
    return 0;
}

int rho_score_residual_dense(const float *q, int m, const uint8_t *codes, const uint8_t *signs,
                             const float *norms, const float *res_scale, int64_t n, int d, int bits,
                             uint64_t seed, double *logits)
{
    double lv[16], th[15];
    int8_t *s;
    double *z;
    int64_t k;
    int i, j, b1 = bits - 1;
    double rd = sqrt((double)d);
    if (!valid_dim(d) || d < 8 || bits < 2 || bits > 5 || n < 0 || m < 0) return -1;
    if ((int64_t)b1 * d % 8) return -1;
    rho_lloyd_max(b1, lv, th, NULL, NULL);
    s = (int8_t *)malloc((size_t)d);
    z = (double *)malloc(sizeof(double) * (size_t)d);
    rho_signs(seed, d, s);
    for (k = 0; k < n; ++k) {
        const uint8_t *crow = codes + k * (b1 * d / 8);
        const uint8_t *srow = signs + k * (d / 8);
        double a = (double)norms[k] / d, sr = (double)res_scale[k] / rd;
        for (i = 0; i < d; ++i) z[i] = lv[get_field(crow, i, b1)] * a + (get_field(srow, i, 1) ? sr : -sr);
        rho_fwht(z, d);
        for (i = 0; i < d; ++i) z[i] *= s[i];
        for (j = 0; j < m; ++j) {
            double acc = 0.0;
            for (i = 0; i < d; ++i) acc += (double)q[(int64_t)j * d + i] * z[i];
            logits[(int64_t)j * n + k] = acc;
        }
    }
    free(z);
    free(s);
    return 0;
}
