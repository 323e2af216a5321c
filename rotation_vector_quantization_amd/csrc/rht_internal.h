// rht_internal.h -- shared between the ABI layer (rht_api.cpp) and the HIP
// kernels (rht_kernels.hip).  Not installed, not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rht {

constexpr int kMinD = 16;
constexpr int kMaxD = 4096;

// What a quantize launch computes.
enum Kind : int {
    kMse = 0,        // b-bit Lloyd-Max codes + ||x||
    kDriveBiased,    // 1-bit signs + ||Pi x||_1 / d
    kDriveUnbiased,  // 1-bit signs + ||x||^2 / ||Pi x||_1
    kResidual,       // (b-1)-bit codes + residual signs + ||x|| + S_r
    kEden,           // b-bit Lloyd-Max codes + S = d ||x||^2 / <c, H D x>
};

// Kernel arguments are passed by value (well under the 4 KiB kernarg limit).
// Codebook and rotation signs travel with every launch, so the library keeps
// no device state.
struct QuantArgs {
    const void *x;
    uint8_t *codes;      // MSE / stage-1 codes, or the DRIVE sign bits
    uint8_t *signs;      // residual sign plane
    float *scale;        // ||x|| (MSE, residual) or S (DRIVE, EDEN)
    float *res_scale;    // S_r (residual)
    int64_t n;
    float lev[16];       // fp32 Lloyd-Max levels of the code width
    float thr[16];       // fp32 thresholds (2^cb - 1 used)
    uint32_t dsign[kMaxD / 32];  // bit i set <=> D_ii = -1
};

struct DequantArgs {
    const uint8_t *codes;
    const uint8_t *signs;
    const float *scale;
    const float *res_scale;
    void *y;
    int64_t n;
    float lev[16];
    uint32_t dsign[kMaxD / 32];
};

struct ScoreArgs {
    const float *q;
    const uint8_t *codes;    // MSE codes, sign bits, or the residual chain's stage-1 codes
    const float *norms;      // ||x|| (MSE, residual) or S (sign codes)
    const uint8_t *signs;    // residual sign plane
    const float *res_scale;  // S_r
    float *logits;
    int64_t n;
    int m;
    float key_mult;          // per-key factor = norms[k] * key_mult (1/d, or 1/sqrt(d) for sign codes)
    int exact;               // nonzero: every level is exact in fp16 (sign codes)
    float lev[16];           // levels (sign codes: -1, +1)
    uint32_t dsign[kMaxD / 32];
};

// Attention of m <= 16 queries over coded keys and values, d = 128, key and
// value codes of 2, 3 or 4 bits each.
// One partial record (rotated value sum z[128], running max M, running sum l,
// two pad floats) per (head, chunk, query) in `ws`.
constexpr int kAttnRecord = 132;
constexpr int kAttnMaxQueries = 16;
// Keys per head: the attention kernel addresses a head's code rows with
// 32-bit byte offsets (row * 64 < 2^32).
constexpr int64_t kAttnMaxKeys = int64_t(1) << 26;
// (head, query) rows per call: keeps both attention grids far below 2^32
// work-items per dimension (the partial kernel launches ~64 work-items per
// head, the combine kernel 64 per row).
constexpr int64_t kAttnMaxRows = int64_t(1) << 24;

// Size of the device array rht_attention_noalloc uses in place of a
// workspace (one per device, for the life of the process).
constexpr size_t kAttnScratchBytes = size_t(32) << 20;

struct AttnArgs {
    const float *q;      // [heads][m][128]
    const uint8_t *kc;   // [heads][n][16 kbits]
    const uint8_t *vc;
    const float *kn;     // [heads][n]
    const float *vn;
    float *ws;           // [heads][chunks][m][kAttnRecord]
    float *out;          // [heads][m][128]
    int64_t heads, n;
    int m, chunks;
    int kbits, vbits;    // code widths of keys and values
    float scale;
    float lev_k[16];     // Lloyd-Max levels of the key codes
    float lev_v[16];     // of the value codes
    uint32_t dsign_k[4], dsign_v[4];
};

// Launchers.  The MSE kernels interleave the lanes of a vector in chunks of
// 32/bits coordinates (one code word each) at 1, 2 and 4 bits and give every
// lane a contiguous run of the row at 3 bits; the DRIVE, residual and EDEN
// kernels always use contiguous runs.
// Return hipErrorInvalidValue when no kernel exists for the combination.
hipError_t launch_quantize(int d, bool f16, int bits, Kind kind, const QuantArgs &a, hipStream_t s);
hipError_t launch_dequantize(int d, bool f16out, int bits, Kind kind, const DequantArgs &a, hipStream_t s);
// bits = code width of a.codes; residual: scores the chain of stage-1 codes
// plus the sign plane.
hipError_t launch_score(int d, int bits, bool residual, const ScoreArgs &a, hipStream_t s);
hipError_t launch_attention(const AttnArgs &a, hipStream_t s);
// Device address of the current device's attention scratch array
// (kAttnScratchBytes), looked up on the first call per device.
hipError_t attention_scratch(void **ptr);

// d = 16: one lane per vector, the transform in registers (launch_quantize,
// launch_dequantize and launch_score pick them for that d).
hipError_t launch_quantize_d16(bool f16, int bits, Kind kind, const QuantArgs &a, hipStream_t s);
hipError_t launch_dequantize_d16(bool f16out, int bits, Kind kind, const DequantArgs &a, hipStream_t s);
hipError_t launch_score_d16(int bits, bool residual, const ScoreArgs &a, hipStream_t s);

// The d = 128, fp16, 4-bit MSE encoder and decoder with the H_32 factor on
// MFMA (launch_quantize / launch_dequantize pick them for that case).
hipError_t launch_quantize_kv128(const QuantArgs &a, hipStream_t s);
hipError_t launch_dequantize_kv128(const DequantArgs &a, hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Whether the d = 128, fp16, 4-bit MSE kernels run the H_32 factor of the
// transform on MFMA (default) or as register/DPP butterflies (RHT_HADAMARD=valu).
bool hadamard_on_mfma();

}  // namespace rht
