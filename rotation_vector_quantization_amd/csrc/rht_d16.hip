// rht_d16.hip -- the randomized Hadamard transform, its codes, decoders and
// rotated-domain scoring at d = 16, the smallest row length of the library.
//
// Method: web page "Random-rotation quantization": Pi = H D / sqrt(d) ("Why
// rotation works"), one N(0,1) Lloyd-Max codebook or its finite-d variant for
// every rotated coordinate ("History", EDEN item; "Why rotation works"),
// DRIVE's sign code with its two scales, the residual chain (TurboQuant item)
// and the inner-product decoder ("Three decoders, one rotation").  The
// arithmetic of every step is that of the kernels for d >= 32:
//   y16 = 16 (H D x)_i / ||x||, code = base + [y16 >= 16 t] from the same
//   nearest-level table; S = ||H D x||_1 / (d sqrt(d)) (biased) or
//   ||x||^2 sqrt(d) / ||H D x||_1 (unbiased); S_r = ||r||^2 / ||r||_1 with
//   r = (||x|| / 16) rho16 / sqrt(d); EDEN S = d ||x||^2 / <c, H D x>;
//   decode x^ = D H z, z = c ||x|| / d, +-S / sqrt(d), or
//   c ||x|| / d + S_r sigma / sqrt(d).
//
// Layout: a whole row is 32 (fp16) or 64 (fp32) bytes, so one lane owns one
// vector and H_16 is four butterfly stages on its registers: no cross-lane
// traffic at all.  A row of b-bit codes is 2b bytes (2, 4, 6 or 8: one 16-,
// 32- or 64-bit word, or three 16-bit words at 3 bits), written LSB-first like
// every other d; the lanes of a wave write consecutive rows, so each store
// instruction covers one contiguous run.
#include "rht_device.h"

namespace rht {
namespace {

constexpr int kD = 16;

// Sylvester-ordered H_16 (unnormalized), in place; FIRST: stages already done.
template <int FIRST = 0>
__device__ __forceinline__ void fwht16(float (&v)[kD]) {
#pragma unroll
    for (int h = 1 << FIRST; h < kD; h <<= 1)
#pragma unroll
        for (int i = 0; i < kD; i += 2 * h)
#pragma unroll
            for (int j = i; j < i + h; ++j) {
                const float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
}

// Row `vec` of x with D applied (bit i of dmask set: coordinate i negated);
// returns sum x_i^2.  fp16 rows go through v_dot2_f32_f16, which takes fp16
// subnormals as they are: per pair of coordinates, one instruction applies
// the signs, converts and forms the first butterfly stage (x0 s0 +- x1 s1),
// and the squares are dot products of the raw halves with themselves.  The
// caller then runs the transform from its second stage (fwht16<1>).
template <bool F16>
__device__ __forceinline__ float load_row16(const void *x, int64_t vec, uint32_t dmask, float (&v)[kD]) {
    float ss = 0.0f, ss2 = 0.0f;
    if constexpr (F16) {
        const u32x4_t *row = reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(x) + vec * kD);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const u32x4_t t = __builtin_nontemporal_load(row + c);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int p = 4 * c + k;  // coordinates 2p, 2p + 1
                const uint32_t sw = ((dmask >> (2 * p)) & 1u ? 0xBC00u : 0x3C00u) |
                                    (((dmask >> (2 * p + 1)) & 1u ? 0xBC00u : 0x3C00u) << 16);
                v[2 * p] = dot2(t[k], sw, 0.0f);
                v[2 * p + 1] = dot2(t[k], sw ^ 0x80000000u, 0.0f);
                if (p & 1)
                    ss2 = dot2(t[k], t[k], ss2);
                else
                    ss = dot2(t[k], t[k], ss);
            }
        }
    } else {
        const u32x4_t *row = reinterpret_cast<const u32x4_t *>(static_cast<const float *>(x) + vec * kD);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4_t t = __builtin_nontemporal_load(row + c);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = 4 * c + k;
                // the element goes through a scalar: this compiler's bit_cast of
                // an ext-vector element itself reads the wrong element
                const uint32_t u = t[k];
                const float f = __builtin_bit_cast(float, u);
                if (i & 1)
                    ss2 = fmaf(f, f, ss2);
                else
                    ss = fmaf(f, f, ss);
                v[i] = __builtin_bit_cast(float, u ^ (((dmask >> i) & 1u) << 31));
            }
        }
    }
    return ss + ss2;
}

// A row of CB-bit codes: 2 CB bytes, code i at bits [CB i, CB i + CB).
template <int CB>
__device__ __forceinline__ void store_code_row(uint8_t *codes, int64_t vec, uint64_t w) {
    if constexpr (CB == 1) {
        __builtin_nontemporal_store((uint16_t)w, reinterpret_cast<uint16_t *>(codes) + vec);
    } else if constexpr (CB == 2) {
        __builtin_nontemporal_store((uint32_t)w, reinterpret_cast<uint32_t *>(codes) + vec);
    } else if constexpr (CB == 3) {
        uint16_t *p = reinterpret_cast<uint16_t *>(codes) + 3 * vec;
#pragma unroll
        for (int k = 0; k < 3; ++k) __builtin_nontemporal_store((uint16_t)(w >> (16 * k)), p + k);
    } else {
        __builtin_nontemporal_store(w, reinterpret_cast<uint64_t *>(codes) + vec);
    }
}

template <int CB>
__device__ __forceinline__ uint64_t load_code_row(const uint8_t *codes, int64_t vec) {
    if constexpr (CB == 1) {
        return __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(codes) + vec);
    } else if constexpr (CB == 2) {
        return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(codes) + vec);
    } else if constexpr (CB == 3) {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(codes) + 3 * vec;
        uint64_t w = 0;
#pragma unroll
        for (int k = 0; k < 3; ++k) w |= (uint64_t)__builtin_nontemporal_load(p + k) << (16 * k);
        return w;
    } else {
        return __builtin_nontemporal_load(reinterpret_cast<const uint64_t *>(codes) + vec);
    }
}

// ---------------------------------------------------------------------------
// Encoder.  KIND as for the other row lengths; CB = width of the written
// codes (BITS - 1 for the residual chain, 1 for DRIVE).
template <bool F16, int CB, int KIND>
__global__ __launch_bounds__(kBlock) void k_quantize16(const QuantArgs a) {
    constexpr bool DRIVE = (KIND == kDriveBiased || KIND == kDriveUnbiased);
    constexpr bool RES = KIND == kResidual, EDEN = KIND == kEden;
    __shared__ uint2 lut[DRIVE ? 1 : Lut<kD>::kCells];
    __shared__ float lev16[16];
    if constexpr (!DRIVE) {
        build_lut<Lut<kD>::kCells, Lut<kD>::kOff>(lut, a.thr, (1 << CB) - 1);
        if (threadIdx.x < 16) lev16[threadIdx.x] = 16.0f * a.lev[threadIdx.x];
        __syncthreads();
    }
    const uint32_t dmask = a.dsign[0] & 0xFFFFu;
    const float sqrt_d = 4.0f;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t vec = (int64_t)blockIdx.x * kBlock + threadIdx.x; vec < a.n; vec += stride) {
        float v[kD];
        const float ss = load_row16<F16>(a.x, vec, dmask, v);
        fwht16<F16 ? 1 : 0>(v);
        uint64_t w = 0;
        if constexpr (DRIVE) {
            // bit_i = [(H D x)_i >= 0]
            float l1 = 0.0f;
#pragma unroll
            for (int i = 0; i < kD; ++i) {
                l1 += fabsf(v[i]);
                w |= (uint64_t)(v[i] >= 0.0f ? 1u : 0u) << i;
            }
            float S;
            if constexpr (KIND == kDriveBiased)
                S = l1 / ((float)kD * sqrt_d);
            else
                S = l1 > 0.0f ? ss / (l1 / sqrt_d) : 0.0f;
            store_code_row<1>(a.codes, vec, w);
            a.scale[vec] = S;
        } else {
            const float nrm = sqrtf(ss);
            const float inv16 = ss > 0.0f ? 16.0f / nrm : 0.0f;
            float r2 = 0.0f, r1 = 0.0f, ch = 0.0f;
            uint32_t neg = 0u;
#pragma unroll
            for (int i = 0; i < kD; ++i) {
                const float y16 = v[i] * inv16;
                const uint32_t code = nearest_code<kD>(lut, y16);
                w |= (uint64_t)code << (CB * i);
                if constexpr (RES) {
                    // residual in units of y16; its sign bit, 1 = negative
                    const float rho = y16 - lev16[code];
                    r2 = fmaf(rho, rho, r2);
                    r1 += fabsf(rho);
                    neg |= (__builtin_bit_cast(uint32_t, rho) >> 31) << i;
                } else if constexpr (EDEN) {
                    ch = fmaf(lev16[code], y16, ch);
                }
            }
            store_code_row<CB>(a.codes, vec, w);
            if constexpr (RES) {
                // a zero vector has residual 0 everywhere, whose sign bit is +1
                const uint32_t sbits = ss > 0.0f ? (~neg & 0xFFFFu) : 0xFFFFu;
                __builtin_nontemporal_store((uint16_t)sbits, reinterpret_cast<uint16_t *>(a.signs) + vec);
                a.res_scale[vec] = r1 > 0.0f ? (nrm * (1.0f / 16.0f)) * (r2 / (sqrt_d * r1)) : 0.0f;
            }
            // EDEN: S = d ||x||^2 / <c, H D x> = d ||x|| 256 / <16 c, y16>
            a.scale[vec] = EDEN ? (ch > 0.0f ? (float)kD * nrm * (256.0f / ch) : 0.0f) : nrm;
        }
    }
}

// ---------------------------------------------------------------------------
// Decoder: x^ = D H z.
template <bool F16OUT, int CB, int KIND>
__global__ __launch_bounds__(kBlock) void k_dequantize16(const DequantArgs a) {
    constexpr bool DRIVE = (KIND == kDriveBiased || KIND == kDriveUnbiased);
    __shared__ float slev[16];
    if (threadIdx.x < 16) slev[threadIdx.x] = a.lev[threadIdx.x];
    __syncthreads();
    const uint32_t dmask = a.dsign[0] & 0xFFFFu;
    const float inv_sqrt_d = 0.25f;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t vec = (int64_t)blockIdx.x * kBlock + threadIdx.x; vec < a.n; vec += stride) {
        const uint64_t w = load_code_row<CB>(a.codes, vec);
        const float sc = a.scale[vec];
        float v[kD], alpha;
        if constexpr (DRIVE) {
#pragma unroll
            for (int i = 0; i < kD; ++i) v[i] = (w >> i) & 1u ? 1.0f : -1.0f;
            alpha = sc * inv_sqrt_d;
        } else if constexpr (KIND == kResidual) {
            const uint32_t sb = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(a.signs) + vec);
            const float a0 = sc * (1.0f / kD), s0 = a.res_scale[vec] * inv_sqrt_d;
#pragma unroll
            for (int i = 0; i < kD; ++i)
                v[i] = fmaf(slev[(w >> (CB * i)) & ((1u << CB) - 1u)], a0, (sb >> i) & 1u ? s0 : -s0);
            alpha = 1.0f;
        } else {
#pragma unroll
            for (int i = 0; i < kD; ++i) v[i] = slev[(w >> (CB * i)) & ((1u << CB) - 1u)];
            alpha = sc * (1.0f / kD);
        }
        fwht16(v);
        // D as an XOR on the sign bits of the scaled (and rounded) outputs
        if constexpr (F16OUT) {
            uint32_t o[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const _Float16 lo = (_Float16)(v[2 * k] * alpha), hi = (_Float16)(v[2 * k + 1] * alpha);
                o[k] = ((uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16)) ^
                       ((((dmask >> (2 * k)) & 1u) << 15) | (((dmask >> (2 * k + 1)) & 1u) << 31));
            }
            u32x4_t *row = reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(a.y) + vec * kD);
            __builtin_nontemporal_store(u32x4_t{o[0], o[1], o[2], o[3]}, row);
            __builtin_nontemporal_store(u32x4_t{o[4], o[5], o[6], o[7]}, row + 1);
        } else {
            u32x4_t *row = reinterpret_cast<u32x4_t *>(static_cast<float *>(a.y) + vec * kD);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                uint32_t o[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    o[k] = __builtin_bit_cast(uint32_t, v[4 * c + k] * alpha) ^ (((dmask >> (4 * c + k)) & 1u) << 31);
                __builtin_nontemporal_store(u32x4_t{o[0], o[1], o[2], o[3]}, row + c);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Scoring: logits[j][k] = f_k sum_i (H D q_j)_i C[k][i] with C = c[code]
// (factor ||k|| / d, or S / sqrt(d) for sign codes, as norms[k] * key_mult),
// or, RES, C = (||k|| / d) c[code] + (S_r / sqrt(d)) sigma with no further
// factor.  The block's m <= 64 queries are rotated once into LDS (one thread
// per query); each thread then scores one key against every query, reading
// the same query row in every lane (an LDS broadcast).
template <int CB, bool RES>
__global__ __launch_bounds__(kBlock) void k_score16(const ScoreArgs a) {
    __shared__ float qt[64][kD + 1];
    __shared__ float slev[16];
    if (threadIdx.x < 16) slev[threadIdx.x] = a.lev[threadIdx.x];
    const uint32_t dmask = a.dsign[0] & 0xFFFFu;
    if ((int)threadIdx.x < a.m) {
        float v[kD];
        load_row16<false>(a.q, threadIdx.x, dmask, v);
        fwht16(v);
#pragma unroll
        for (int i = 0; i < kD; ++i) qt[threadIdx.x][i] = v[i];
    }
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t key = (int64_t)blockIdx.x * kBlock + threadIdx.x; key < a.n; key += stride) {
        const uint64_t w = load_code_row<CB>(a.codes, key);
        float b[kD], f;
        if constexpr (RES) {
            const uint32_t sb = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(a.signs) + key);
            const float na = a.norms[key] * (1.0f / kD), nb = a.res_scale[key] * 0.25f;
#pragma unroll
            for (int i = 0; i < kD; ++i)
                b[i] = fmaf(na, slev[(w >> (CB * i)) & ((1u << CB) - 1u)], (sb >> i) & 1u ? nb : -nb);
            f = 1.0f;
        } else {
#pragma unroll
            for (int i = 0; i < kD; ++i) b[i] = slev[(w >> (CB * i)) & ((1u << CB) - 1u)];
            f = a.norms[key] * a.key_mult;
        }
        for (int j = 0; j < a.m; ++j) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < kD; ++i) acc = fmaf(qt[j][i], b[i], acc);
            __builtin_nontemporal_store(acc * f, a.logits + (int64_t)j * a.n + key);
        }
    }
}

template <bool F16, int CB, int KIND>
hipError_t run_q16(const QuantArgs &a, hipStream_t s) {
    static const int per_cu = resident_blocks(k_quantize16<F16, CB, KIND>);
    return launch(k_quantize16<F16, CB, KIND>, dim3(grid_for(a.n, kBlock, per_cu)), dim3(kBlock), s, a);
}

template <int CB, int KIND>
hipError_t run_q16_x(bool f16, const QuantArgs &a, hipStream_t s) {
    return f16 ? run_q16<true, CB, KIND>(a, s) : run_q16<false, CB, KIND>(a, s);
}

template <bool F16OUT, int CB, int KIND>
hipError_t run_dq16(const DequantArgs &a, hipStream_t s) {
    static const int per_cu = resident_blocks(k_dequantize16<F16OUT, CB, KIND>);
    return launch(k_dequantize16<F16OUT, CB, KIND>, dim3(grid_for(a.n, kBlock, per_cu)), dim3(kBlock), s, a);
}

template <int CB, int KIND>
hipError_t run_dq16_x(bool f16out, const DequantArgs &a, hipStream_t s) {
    return f16out ? run_dq16<true, CB, KIND>(a, s) : run_dq16<false, CB, KIND>(a, s);
}

template <int CB, bool RES>
hipError_t run_score16(const ScoreArgs &a, hipStream_t s) {
    static const int per_cu = resident_blocks(k_score16<CB, RES>);
    return launch(k_score16<CB, RES>, dim3(grid_for(a.n, kBlock, per_cu)), dim3(kBlock), s, a);
}

}  // namespace

hipError_t launch_quantize_d16(bool f16, int bits, Kind kind, const QuantArgs &a, hipStream_t s) {
    switch (kind) {
    case kMse:
        switch (bits) {
        case 1: return run_q16_x<1, kMse>(f16, a, s);
        case 2: return run_q16_x<2, kMse>(f16, a, s);
        case 3: return run_q16_x<3, kMse>(f16, a, s);
        case 4: return run_q16_x<4, kMse>(f16, a, s);
        }
        break;
    case kEden:
        switch (bits) {
        case 1: return run_q16_x<1, kEden>(f16, a, s);
        case 2: return run_q16_x<2, kEden>(f16, a, s);
        case 3: return run_q16_x<3, kEden>(f16, a, s);
        case 4: return run_q16_x<4, kEden>(f16, a, s);
        }
        break;
    case kDriveBiased: return run_q16_x<1, kDriveBiased>(f16, a, s);
    case kDriveUnbiased: return run_q16_x<1, kDriveUnbiased>(f16, a, s);
    case kResidual:
        switch (bits) {
        case 2: return run_q16_x<1, kResidual>(f16, a, s);
        case 3: return run_q16_x<2, kResidual>(f16, a, s);
        case 4: return run_q16_x<3, kResidual>(f16, a, s);
        }
        break;
    }
    return hipErrorInvalidValue;
}

hipError_t launch_dequantize_d16(bool f16out, int bits, Kind kind, const DequantArgs &a, hipStream_t s) {
    switch (kind) {
    case kMse:
        switch (bits) {
        case 1: return run_dq16_x<1, kMse>(f16out, a, s);
        case 2: return run_dq16_x<2, kMse>(f16out, a, s);
        case 3: return run_dq16_x<3, kMse>(f16out, a, s);
        case 4: return run_dq16_x<4, kMse>(f16out, a, s);
        }
        break;
    case kDriveBiased:
    case kDriveUnbiased: return run_dq16_x<1, kDriveBiased>(f16out, a, s);
    case kResidual:
        switch (bits) {
        case 2: return run_dq16_x<1, kResidual>(f16out, a, s);
        case 3: return run_dq16_x<2, kResidual>(f16out, a, s);
        case 4: return run_dq16_x<3, kResidual>(f16out, a, s);
        }
        break;
    case kEden:  // EDEN codes decode as MSE codes (the caller passes kMse)
        break;
    }
    return hipErrorInvalidValue;
}

hipError_t launch_score_d16(int bits, bool residual, const ScoreArgs &a, hipStream_t s) {
    if (residual) {
        switch (bits) {
        case 1: return run_score16<1, true>(a, s);
        case 2: return run_score16<2, true>(a, s);
        case 3: return run_score16<3, true>(a, s);
        }
        return hipErrorInvalidValue;
    }
    switch (bits) {
    case 1: return run_score16<1, false>(a, s);
    case 2: return run_score16<2, false>(a, s);
    case 3: return run_score16<3, false>(a, s);
    case 4: return run_score16<4, false>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace rht
