/*
 * rht.h -- C ABI of librht, randomized-Hadamard (random-rotation) vector
 * quantization on AMD Instinct MI355X (gfx950).
 *
 * Method: the web page "Random-rotation quantization" (brain.bigb.es).  Every
 * vector x of length d is rotated by Pi = H D / sqrt(d) (D = diagonal of
 * seeded +-1 signs, H the Sylvester-ordered Hadamard matrix, applied as a fast
 * Walsh-Hadamard transform), each rotated coordinate is quantized
 * independently with one fixed codebook, and the decoder applies Pi^T
 * ("intro", steps 1-3; "Why rotation works": randomized Hadamard transform).
 *
 * Conventions shared by every call below
 *   - Array arguments are DEVICE pointers owned by the caller (for example
 *     torch tensors); the library never allocates, frees or keeps them.
 *   - Row-major: one contiguous row per vector.  n = number of vectors (rows),
 *     d = row length, a power of two with 16 <= d <= 4096.
 *   - Codes are an LSB-first bitstream per row: coordinate i occupies bits
 *     [b*i, b*i + b) of its row; a row of b-bit codes is b*d/8 bytes.
 *   - Every device pointer must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Kernels are queued on
 *     it and the call returns before they finish; the caller synchronizes.
 *   - Arguments are validated on the host before anything is queued, in this
 *     order: counts (RHT_E_COUNT), d (RHT_E_DIM), bits (RHT_E_BITS), mode
 *     (RHT_E_MODE), element type (RHT_E_DTYPE); then n == 0 (or m == 0)
 *     returns RHT_OK without touching any pointer; then NULL pointers
 *     (RHT_E_NULL) and alignment (RHT_E_ALIGN).  The first failing check is
 *     returned and nothing is launched.  A failed launch comes back as
 *     RHT_E_DEVICE: the status of the call's own launches, not an error
 *     some earlier HIP call left pending on the thread (that stays for the
 *     caller's hipGetLastError).  No call prints, aborts or throws.
 *   - The same (d, bits, seed) must be used to encode and to decode.  The
 *     rotation depends on the seed only (signs = top bits of the SplitMix64
 *     stream started at `seed`, see rht_signs), never on the data.
 *   - Inputs must be finite and ||x||^2 must be a normal fp32 number or 0;
 *     other inputs give unspecified (but memory-safe) results.  Outputs must
 *     not alias inputs.  Calls on different streams may run concurrently.
 */
#ifndef RHT_H
#define RHT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RHT_ABI_VERSION 6

typedef enum {
    RHT_OK = 0,
    RHT_E_NULL = 1,    /* a required pointer is NULL */
    RHT_E_DIM = 2,     /* d not a power of two, or outside the supported range */
    RHT_E_BITS = 3,    /* bits outside the range of the call */
    RHT_E_DTYPE = 4,   /* unknown element type */
    RHT_E_MODE = 5,    /* unknown mode, or a mode that does not allow these bits */
    RHT_E_ALIGN = 6,   /* a device pointer is not 16-byte aligned */
    RHT_E_COUNT = 7,   /* n < 0, or m outside [0, 64] */
    RHT_E_DEVICE = 8,  /* the HIP runtime reported an error (bad stream/pointer, launch) */
    RHT_E_WORKSPACE = 9 /* workspace smaller than the call needs */
} rht_status;

typedef enum { RHT_F32 = 0, RHT_F16 = 1 } rht_dtype;

typedef enum {
    /* EDEN / TurboQuant MSE code ("History", EDEN and TurboQuant items;
       "Three decoders, one rotation", MSE decoder): y = H D x / ||x|| (each
       coordinate ~ N(0,1)), code_i = index of the nearest N(0,1) Lloyd-Max
       level (ties go to the upper level), scalar = ||x||_2.  bits 1..4. */
    RHT_SCALE_NORM = 0,
    /* DRIVE 1-bit code ("History", DRIVE item; "Three decoders", mean
       decoder): bit_i = [(Pi x)_i >= 0], scalar S = ||Pi x||_1 / d (biased,
       MSE-optimal).  bits must be 1. */
    RHT_SCALE_SIGN_BIASED = 1,
    /* Same bits, S = ||x||_2^2 / ||Pi x||_1 (unbiased; 0 when ||Pi x||_1 = 0). */
    RHT_SCALE_SIGN_UNBIASED = 2,
    /* EDEN-style unbiased scale for the MSE code ("History", EDEN item; "Bias
       vs unbiasedness"): the codes of RHT_SCALE_NORM, scalar S = d ||x||^2 /
       <c[code], H D x> (0 when that is 0), so the decoder's x^ = D H (c S / d)
       has <x^, x> = ||x||^2.  bits 1..4; at 1 bit it equals the unbiased sign
       code.  Decodes, scores and attends exactly like RHT_SCALE_NORM codes
       with S in place of ||x||. */
    RHT_SCALE_EDEN = 3,
    /* RHT_SCALE_NORM with the exact finite-d codebook ("Why rotation works":
       a rotated coordinate follows a Beta law, not N(0,1)): the Lloyd-Max
       quantizer of y = sqrt(d) t, (1 + t)/2 ~ Beta((d-1)/2, (d-1)/2), see
       rht_codebook_beta.  bits 1..4; decode with the same mode. */
    RHT_SCALE_NORM_BETA = 4
} rht_mode;

/* Encode n vectors.
 *   x      [n][d] elements of type xt (fp32 or fp16), read only.
 *   codes  [n][bits*d/8] bytes, written.
 *   scale  [n] fp32, written: ||x||_2 (RHT_SCALE_NORM) or S (sign modes, RHT_SCALE_EDEN).
 *   bits   1..4 for RHT_SCALE_NORM and RHT_SCALE_EDEN; exactly 1 for the sign modes.
 * Passage: "intro" steps 1-2; "History" (EDEN normalization and Lloyd-Max
 * codebook; DRIVE signs and scale). */
rht_status rht_quantize(const void *x, rht_dtype xt, int64_t n, int32_t d, int32_t bits,
                        rht_mode mode, uint64_t seed, uint8_t *codes, float *scale, void *stream);

/* Decode n vectors encoded by rht_quantize with the same (d, bits, mode, seed).
 *   RHT_SCALE_NORM: y = Pi^T (c[code] * ||x|| / sqrt(d)) = D H (c[code] * ||x|| / d).
 *   sign modes:     y = S * Pi^T sigma, sigma_i = +1 for a set bit, else -1.
 *   y [n][d] of type yt, written (fp16 output is rounded to nearest even).
 * Passage: "intro" step 3; "Three decoders, one rotation" (MSE and mean decoders). */
rht_status rht_dequantize(const uint8_t *codes, const float *scale, int64_t n, int32_t d,
                          int32_t bits, rht_mode mode, uint64_t seed, void *y, rht_dtype yt,
                          void *stream);

/* Residual chain with `bits` bits per coordinate in total, 2..4 ("History",
 * TurboQuant item; "Bias vs unbiasedness"): stage 1 is the (bits-1)-bit MSE
 * code (identical to rht_quantize with bits-1); the rotated-domain residual
 * r = Pi (x - x~) gets one sign bit per coordinate, sbit_i = [r_i >= 0], and
 * DRIVE's unbiased scale S_r = ||r||_2^2 / ||r||_1 (0 when ||r||_1 = 0).
 *   x         [n][d] of type xt.
 *   codes     [n][(bits-1)*d/8] written;  signs [n][d/8] written;
 *   norms     [n] fp32 ||x||_2 written;   res_scale [n] fp32 S_r written.
 * (bits-1)*d/8 code bytes per row; bits = 4 uses 3-bit codes. */
rht_status rht_residual_quantize(const void *x, rht_dtype xt, int64_t n, int32_t d, int32_t bits,
                                 uint64_t seed, uint8_t *codes, uint8_t *signs, float *norms,
                                 float *res_scale, void *stream);

/* Decode the residual chain: y = Pi^T (c[code] ||x|| / sqrt(d) + S_r sigma)
 * = D H (c[code] ||x|| / d + S_r sigma / sqrt(d)).  Arguments as above;
 * y [n][d] of type yt written. */
rht_status rht_residual_dequantize(const uint8_t *codes, const uint8_t *signs, const float *norms,
                                   const float *res_scale, int64_t n, int32_t d, int32_t bits,
                                   uint64_t seed, void *y, rht_dtype yt, void *stream);

/* Score queries against MSE-coded keys without decoding them ("Three
 * decoders, one rotation", inner-product decoder: <q, Pi^T z> = <Pi q, z>):
 *   logits[j][k] = <q_j, dequant(k_k)> = (||k_k|| / d) * sum_i (H D q_j)_i c[code_{k,i}]
 * H D q_j is formed once per query.  Raw fp32 inner products: no 1/sqrt(d)
 * attention scale, no softmax.
 *   q      [m][d] fp32, 0 <= m <= 64;  codes [n][bits*d/8], norms [n] fp32 as
 *          written by rht_quantize(..., RHT_SCALE_NORM, seed, ...).
 *   logits [m][n] fp32 written.  d a power of two in [16, 4096]; bits 1..4. */
rht_status rht_score(const float *q, int32_t m, const uint8_t *codes, const float *norms, int64_t n,
                     int32_t d, int32_t bits, uint64_t seed, float *logits, void *stream);

/* Inner products with sign-coded keys ("Three decoders, one rotation",
 * inner-product decoder: <q, x> from <Pi q, sign(Pi x)> with a normalizing
 * scalar).  For bits and S written by rht_quantize(..., RHT_SCALE_SIGN_BIASED
 * or RHT_SCALE_SIGN_UNBIASED, seed, ...) with bits = 1, the logits are the
 * inner products with the mean decoder's vectors, x^ = S D H sigma / sqrt(d):
 *   logits[j][k] = (S_k / sqrt(d)) * sum_i (H D q_j)_i sigma_{k,i},  sigma = +-1.
 * With the unbiased scale their mean over rotation seeds is <q_j, x_k>.
 *   q [m][d] fp32, 0 <= m <= 64; bits [n][d/8]; scale [n] fp32;
 *   logits [m][n] fp32 written.  d a power of two in [16, 4096]. */
rht_status rht_score_sign(const float *q, int32_t m, const uint8_t *bits, const float *scale, int64_t n,
                          int32_t d, uint64_t seed, float *logits, void *stream);

/* Inner products with residual-chain-coded keys ("History", TurboQuant item;
 * "Bias vs unbiasedness": b-1 bit MSE code plus a 1-bit code of the residual):
 *   logits[j][k] = (||x_k|| / d) sum_i (H D q_j)_i c[code_{k,i}]
 *                + (S_r,k / sqrt(d)) sum_i (H D q_j)_i sigma_{k,i}
 * = <q_j, x^_k> for the vectors rht_residual_dequantize returns.  Arguments
 * as written by rht_residual_quantize (total bits 2..4); q [m][d] fp32,
 * 0 <= m <= 64; logits [m][n] fp32 written; d a power of two in [16, 4096]. */
rht_status rht_residual_score(const float *q, int32_t m, const uint8_t *codes, const uint8_t *signs,
                              const float *norms, const float *res_scale, int64_t n, int32_t d, int32_t bits,
                              uint64_t seed, float *logits, void *stream);

/* Attention over MSE-coded keys and values, computed in the rotated domains
 * (page "Attn-rot: TurboQuant lite in llama.cpp", opening section: the keys
 * and values of the KV cache are rotated and quantized; "Three decoders, one
 * rotation": logits come from <Pi q, code>, and since Pi^T is linear the
 * weighted sum of decoded values is one inverse rotation of the weighted sum
 * of their codes).  For every head h and query i:
 *   out[h][i] = sum_j softmax_j(scale * <q[h][i], k~[h][j]>) v~[h][j]
 * where k~, v~ are the vectors rht_dequantize would decode (keys with seed_k
 * and k_bits, values with seed_v and v_bits).  No mask; scale is applied as
 * given (e.g. 1/sqrt(d)).  Keys and values take their own code widths ("Random-
 * rotation quantization", "Practical use in llama.cpp": separate K and V cache
 * types, e.g. 4-bit keys with 3-bit values).
 *   q          [heads][m][d] fp32, 1 <= m <= 16, heads * m <= 2^24
 *              (RHT_E_COUNT otherwise).
 *   k_codes    [heads][n][k_bits*d/8], v_codes [heads][n][v_bits*d/8] and
 *              k_norms, v_norms [heads][n] fp32, as written by
 *              rht_quantize(..., RHT_SCALE_NORM or RHT_SCALE_EDEN, seed, ...).
 *   out        [heads][m][d] fp32, written.
 *   workspace  device scratch of at least rht_attention_workspace_bytes(heads,
 *              m, n, d) bytes, owned by the caller; its contents on entry are
 *              ignored and on return unspecified.  Calls that may run at the
 *              same time must not share it.
 *   d = 128 only; k_bits and v_bits 2, 3 or 4 (RHT_E_BITS otherwise).
 *   1 <= n <= 2^26 keys per head when heads > 0
 *   (RHT_E_COUNT otherwise); heads = 0 is a no-op.
 * Returns RHT_E_WORKSPACE (after the other checks) when workspace_bytes is
 * too small. */
rht_status rht_attention(const float *q, int32_t m, const uint8_t *k_codes, const float *k_norms,
                         const uint8_t *v_codes, const float *v_norms, int64_t heads, int64_t n,
                         int32_t d, int32_t k_bits, int32_t v_bits, uint64_t seed_k, uint64_t seed_v,
                         float scale, float *out, void *workspace, size_t workspace_bytes, void *stream);

/* Device workspace bytes rht_attention needs for these sizes; 0 when
 * rht_attention would reject them or has nothing to do.  Host-only. */
size_t rht_attention_workspace_bytes(int64_t heads, int32_t m, int64_t n, int32_t d);

/* rht_attention without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Arguments, validation order, kernels and results are
 * those of rht_attention; the partial records go to a device array inside the
 * library instead, RHT_ATTENTION_NOALLOC_MAX_BYTES bytes, one per device,
 * held from the first call on that device until the process ends.  The call
 * itself allocates nothing: no hipMalloc, no hipFree, no allocating library
 * routine.
 *   Returns RHT_E_WORKSPACE (after the other checks) when these sizes need
 *   more than RHT_ATTENTION_NOALLOC_MAX_BYTES, i.e. when
 *   rht_attention_workspace_bytes(heads, m, n, d) exceeds it (for example
 *   heads * m > 63550 with one key chunk per head).
 *   Every call on a device shares that device's array, and calls whose work
 *   can overlap on one device (different streams, or host threads queueing at
 *   once) race on it and give wrong results: serialize them, for example on
 *   one stream.  No array contents need clearing: each call writes every
 *   record it reads.  RHT_E_DEVICE when the array's device address cannot be
 *   looked up. */
#define RHT_ATTENTION_NOALLOC_MAX_BYTES ((size_t)32 << 20)
rht_status rht_attention_noalloc(const float *q, int32_t m, const uint8_t *k_codes, const float *k_norms,
                                 const uint8_t *v_codes, const float *v_norms, int64_t heads, int64_t n,
                                 int32_t d, int32_t k_bits, int32_t v_bits, uint64_t seed_k, uint64_t seed_v,
                                 float scale, float *out, void *stream);

/* ---- host-side helpers: HOST pointers, synchronous, no GPU needed ---- */

/* The fp32 N(0,1) Lloyd-Max codebook the kernels use ("History", EDEN item):
 * levels[2^bits] ascending, thresholds[2^bits - 1] = midpoints of neighbouring
 * levels, the middle one exactly 0.  bits 1..4.  Either pointer may be NULL. */
rht_status rht_codebook(int32_t bits, float *levels, float *thresholds);

/* The fp32 exact finite-d codebook RHT_SCALE_NORM_BETA uses for (bits, d):
 * the Lloyd-Max quantizer of sqrt(d) times a coordinate of a uniformly
 * rotated unit vector ("Why rotation works": a Beta marginal), levels[2^bits]
 * ascending, thresholds[2^bits - 1] midpoints, the middle one 0.  bits 1..4,
 * d a power of two in [16, 4096].  Either pointer may be NULL. */
rht_status rht_codebook_beta(int32_t bits, int32_t d, float *levels, float *thresholds);

/* The diagonal D of the rotation for (seed, d): signs[i] = -1 when the top bit
 * of the i-th SplitMix64 output started from state `seed` is set, else +1.
 * d >= 1. */
rht_status rht_signs(uint64_t seed, int32_t d, int8_t *signs);

/* Static string naming a status; never NULL. */
const char *rht_status_str(rht_status status);

/* RHT_ABI_VERSION of the loaded library. */
int32_t rht_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RHT_H */
