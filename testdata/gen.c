/*
 * gen.c -- seeded, counter-based synthetic inputs shared by the tests, the
 * benchmark and the smoke check.  It holds none of the quantizer's
 * arithmetic: it only draws the input vectors.
 *
 * Definitions (any row range can be drawn on its own, in any order):
 *   mix64(z)         SplitMix64 finalizer (Steele, Lea, Flood 2014).
 *   draw(key, i)     mix64(key + (i + 1) * 0x9E3779B97F4A7C15), the i-th
 *                    output of a SplitMix64 stream whose state starts at key.
 *   unif(key, i)     (draw(key, i) >> 11) * 2^-53, in [0, 1).
 *   normal(key, i)   Box-Muller on the pair j = i >> 1:
 *                    r = sqrt(-2 ln(1 - unif(key, 2j))), a = 2 pi unif(key, 2j+1);
 *                    even i -> r cos a, odd i -> r sin a.
 *   subkey(seed, t)  mix64(seed ^ mix64(t + 1)); t = 1 values, 2 outlier
 *                    channels, 3 per-vector log-normal factors, 4 Student-t
 *                    denominators.
 * A value is formed in fp64, rounded to fp32, and for fp16 outputs rounded
 * again fp32 -> fp16 (round-to-nearest-even).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GEN_PI 3.14159265358979323846

static uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * 0x9E3779B97F4A7C15ULL); }

static double unif(uint64_t key, uint64_t i) { return (double)(draw(key, i) >> 11) * 0x1p-53; }

static double normal(uint64_t key, uint64_t i)
{
    uint64_t j = i >> 1;
    double u1 = 1.0 - unif(key, 2 * j);
    double u2 = unif(key, 2 * j + 1);
    double r = sqrt(-2.0 * log(u1));
    double a = 2.0 * GEN_PI * u2;
    return (i & 1) ? r * sin(a) : r * cos(a);
}

uint64_t tdg_subkey(uint64_t seed, uint64_t tag) { return mix64(seed ^ mix64(tag + 1)); }

double tdg_unif(uint64_t key, uint64_t i) { return unif(key, i); }
double tdg_normal(uint64_t key, uint64_t i) { return normal(key, i); }

/* fp32 -> fp16 bits, round-to-nearest-even (IEEE-754 binary16). */
static uint16_t f32_to_f16(float f)
{
    uint32_t x;
    uint32_t sign, e, m;
    memcpy(&x, &f, 4);
    sign = (x >> 16) & 0x8000u;
    e = (x >> 23) & 0xFFu;
    m = x & 0x7FFFFFu;
    if (e == 0xFF) return (uint16_t)(sign | 0x7C00u | (m ? 0x200u : 0u));
    {
        int ue = (int)e - 127; /* unbiased exponent */
        if (ue > 15) return (uint16_t)(sign | 0x7C00u);
        if (ue >= -14) {
            /* normal half: keep 10 mantissa bits, round the 13 dropped ones */
            uint32_t hm = m >> 13, rest = m & 0x1FFFu;
            uint32_t h = ((uint32_t)(ue + 15) << 10) | hm;
            if (rest > 0x1000u || (rest == 0x1000u && (hm & 1u))) h += 1; /* may carry into exp */
            return (uint16_t)(sign | h);
        } else {
            /* subnormal half: value = full * 2^(ue-23), unit 2^-24 */
            uint32_t full = m | 0x800000u;
            int shift = -ue - 14 + 13; /* bits dropped below the 2^-24 unit */
            uint32_t hm, rest, half;
            if (e == 0 || shift > 24) return (uint16_t)sign;
            hm = full >> shift;
            rest = full & ((1u << shift) - 1u);
            half = 1u << (shift - 1);
            if (rest > half || (rest == half && (hm & 1u))) hm += 1;
            return (uint16_t)(sign | hm);
        }
    }
}

uint16_t tdg_f32_to_f16(float f) { return f32_to_f16(f); }

/* Pick `count` distinct channels of [0, d) by a seeded Fisher-Yates shuffle. */
void tdg_pick_channels(uint64_t seed, int d, int count, int32_t *out)
{
    int32_t *p = (int32_t *)malloc(sizeof(int32_t) * (size_t)d);
    uint64_t key = tdg_subkey(seed, 2);
    int i;
    for (i = 0; i < d; ++i) p[i] = i;
    for (i = d - 1; i > 0; --i) {
        int j = (int)(unif(key, (uint64_t)(d - 1 - i)) * (i + 1));
        int32_t t = p[i];
        if (j > i) j = i;
        p[i] = p[j];
        p[j] = t;
    }
    for (i = 0; i < count; ++i) out[i] = p[i];
    free(p);
}

typedef struct {
    int kind;            /* 0: Gaussian with outlier channels, 1: Student-t (nu = 3) */
    uint64_t seed;
    int64_t row0, nrows;
    int d;
    const int32_t *channels;
    int nchannels;
    double mult;         /* outlier channel multiplier */
    double lognorm_sigma;/* > 0: each vector times exp(sigma * g), g ~ N(0,1) */
    int out_f16;
    void *out;
} gen_job;

typedef struct {
    const gen_job *job;
    int64_t r_begin, r_end;
} gen_part;

static void *gen_worker(void *arg)
{
    const gen_part *pt = (const gen_part *)arg;
    const gen_job *jb = pt->job;
    uint64_t kx = tdg_subkey(jb->seed, 1), kg = tdg_subkey(jb->seed, 3), kt = tdg_subkey(jb->seed, 4);
    double *mul = (double *)malloc(sizeof(double) * (size_t)jb->d);
    int64_t r;
    int j, c;
    for (j = 0; j < jb->d; ++j) mul[j] = 1.0;
    for (c = 0; c < jb->nchannels; ++c) mul[jb->channels[c]] = jb->mult;
    for (r = pt->r_begin; r < pt->r_end; ++r) {
        int64_t grow = jb->row0 + r;
        double vf = jb->lognorm_sigma > 0.0 ? exp(jb->lognorm_sigma * normal(kg, (uint64_t)grow)) : 1.0;
        for (j = 0; j < jb->d; ++j) {
            uint64_t idx = (uint64_t)grow * (uint64_t)jb->d + (uint64_t)j;
            double v;
            float f;
            if (jb->kind == 1) {
                double z1 = normal(kt, 3 * idx), z2 = normal(kt, 3 * idx + 1), z3 = normal(kt, 3 * idx + 2);
                v = normal(kx, idx) / sqrt((z1 * z1 + z2 * z2 + z3 * z3) / 3.0);
            } else {
                v = normal(kx, idx) * mul[j] * vf;
            }
            f = (float)v;
            if (jb->out_f16)
                ((uint16_t *)jb->out)[r * jb->d + j] = f32_to_f16(f);
            else
                ((float *)jb->out)[r * jb->d + j] = f;
        }
    }
    free(mul);
    return NULL;
}

int tdg_generate(int kind, uint64_t seed, int64_t row0, int64_t nrows, int d,
                 const int32_t *channels, int nchannels, double mult, double lognorm_sigma,
                 int out_f16, void *out, int nthreads)
{
    gen_job jb;
    gen_part parts[256];
    pthread_t th[256];
    int t;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nrows < (int64_t)nthreads * 64) nthreads = 1;
    jb.kind = kind; jb.seed = seed; jb.row0 = row0; jb.nrows = nrows; jb.d = d;
    jb.channels = channels; jb.nchannels = nchannels; jb.mult = mult;
    jb.lognorm_sigma = lognorm_sigma; jb.out_f16 = out_f16; jb.out = out;
    for (t = 0; t < nthreads; ++t) {
        parts[t].job = &jb;
        parts[t].r_begin = nrows * t / nthreads;
        parts[t].r_end = nrows * (t + 1) / nthreads;
    }
    if (nthreads == 1) {
        gen_worker(&parts[0]);
        return 0;
    }
    for (t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, gen_worker, &parts[t]);
    for (t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    return 0;
}
