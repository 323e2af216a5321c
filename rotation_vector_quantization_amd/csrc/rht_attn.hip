// rht_attn.hip -- attention of a few queries over MSE-coded keys and values
// (d = 128; keys and values each with 2-, 3- or 4-bit codes), computed in the
// rotated domains.
//
// Method: page "Attn-rot: TurboQuant lite in llama.cpp" (opening section: the
// keys and values of the KV cache are rotated and quantized and attention
// runs on them) and page "Random-rotation quantization", "Three decoders, one
// rotation": an inner product with a decoded vector is an inner product of
// the rotated query with the codes, <q, D H c ||k|| / d> = (||k|| / d) <H D q, c>,
// and because Pi^T is linear the weighted sum of decoded values is one inverse
// transform of the weighted sum of their codes:
//     out = sum_j p_j D_v H (c_vj ||v_j|| / d) = D_v H (sum_j p_j (||v_j|| / d) c_vj).
//
// Work split (flash-decoding): the keys of each head are cut into chunks of
// 32-key tiles, one wavefront per (head, chunk).  A wave keeps an online
// softmax (running max M, running sum l, rotated value sum z) and writes one
// partial record per query; a second kernel merges a head's partials and
// applies D_v H once per query.
//
// Both contractions run on v_mfma_f32_16x16x32_f16.  fp32 accuracy comes
// from splitting every operand into fp16 hi + lo parts (x = hi + lo to about
// 2^-22 relative); the products hi*hi, hi*lo and lo*hi are summed in fp32.
//   logits:  C[key][query] = sum_k A[key][k] B[k][query], A = code levels of
//            16 keys (hi/lo from a table indexed by code byte), B = H D_k q
//            scaled by a power of two into fp16 range.
//   values:  z^T[coord][query] += sum_key Cv^T[coord][key] P[key][query],
//            P = p_j ||v_j|| times a running power of two; the accumulator
//            layout of the logits tiles is exactly the B layout P needs.
// Three column layouts, by the number of queries per head m (QueryOps):
// m <= 16 one column per query; m <= 8 the hi and lo parts of the queries and
// of P in separate columns and {hi, lo} level pairs in the K dimension; m <= 4
// also a coordinate parity in the value columns, so the value codes are used
// as stored instead of transposed.
// Lane layout of the 16x16x32 instruction (lane l, g = l / 16): A holds
// A[l % 16][8 g + t], B holds B[8 g + t][l % 16], C holds C[4 g + r][l % 16].
//
// Code widths (page "Random-rotation quantization", "Practical use in
// llama.cpp": the K and V caches take their own code types, e.g. 4-bit keys
// with 3-bit values).  Codes narrower than 4 bits are widened to one code per
// nibble as they arrive (key pieces in registers, value rows on their way
// into LDS), so everything after that sees the 4-bit layout: a byte holds two
// neighbouring codes.  The level tables are indexed by such a byte and built
// from each operand's own codebook; keys and values share one table when
// their widths agree.
#include "rht_device.h"

#include <atomic>
#include <mutex>

namespace rht {
namespace {

// Partial records of rht_attention_noalloc (which takes no workspace): one
// array per device, in the code object, shared by every such call on that
// device.  Host code never uses its name as an address; attention_scratch()
// looks up each device's copy once with hipGetSymbolAddress.
static __device__ __align__(256) float scratch[kAttnScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

constexpr int kAD = 128;           // coordinates per vector
constexpr int kVRow = 80;          // LDS row stride of a staged value tile (bank spread)
// Blocks of RHT_ATTN_WAVES wavefronts share one copy of the level tables; one
// block fills a CU up to the register limit (3 waves per SIMD).
#ifndef RHT_ATTN_WAVES
#define RHT_ATTN_WAVES 12
#endif
constexpr int kAWaves = RHT_ATTN_WAVES;
constexpr int kABlock = 64 * kAWaves;

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma1632(u32x4_t a, u32x4_t b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

// fp16 hi/lo split of two floats, packed as (hi0 | hi1 << 16, lo0 | lo1 << 16).
__device__ __forceinline__ uint2 split2(float x0, float x1) {
    const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
    const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
    return make_uint2((uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16),
                      (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16));
}

// 2^e as a float for -126 <= e <= 127.
__device__ __forceinline__ float pow2i(int e) { return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23); }

// Exponent e with 2^(e-1) <= x < 2^e for a positive normal x.
__device__ __forceinline__ int exponent_above(float x) {
    return (int)((__builtin_bit_cast(uint32_t, x) >> 23) & 0xFFu) - 126;
}

// Unnormalized Hadamard transform of a 128-vector held two coordinates per
// lane (lane l: coordinates 2l, 2l+1); exact butterflies, true values.
__device__ __forceinline__ void fwht128_pairs(float &v0, float &v1, uint32_t lane) {
    const float a = v0 + v1, b = v0 - v1;
    v0 = a;
    v1 = b;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const float p0 = __shfl_xor(v0, m), p1 = __shfl_xor(v1, m);
        v0 = (lane & m) ? p0 - v0 : v0 + p0;
        v1 = (lane & m) ? p1 - v1 : v1 + p1;
    }
}

// Maximum over the four 16-lane rows of the wave, in every lane (the
// butterflies across lanes l ^ 16 and l ^ 32) without a trip through LDS.
// v_permlane16_swap exchanges the odd rows of its first register with the
// even rows of its second: applied to two copies of x it leaves rows
// (0, 0, 2, 2) of x in one and rows (1, 1, 3, 3) in the other;
// v_permlane32_swap does the same with halves of the wave.  Written in asm
// with both registers as in-out operands (the s_nop covers the wait states
// between a VALU write and the swap's read).
__device__ __forceinline__ float max_over_rows(float x) {
    float a = x, b = x;
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    x = fmaxf(a, b);
    a = x;
    b = x;
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return fmaxf(a, b);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

// Global loads of one 32-key tile for a lane (KB, VB: key and value code
// widths; a row of b-bit codes is 16 b bytes).  Keys: the piece of keys
// key0 + l%16 and key0 + 16 + l%16 holding coordinates 32g .. 32g + 31 (4 KB
// bytes each).  Values, 4-bit: the lane's two 16-byte pieces of the 32 x
// 64-byte value tile (chunks l and 64 + l); narrower: half l%2 of the row of
// key key0 + l/2 (8 VB bytes).  One norm (lanes 0-31: key norm of key0 + l,
// lanes 32-63: value norm of key0 + l - 32).  Offsets are 32-bit from
// per-head bases; FULL tiles need no clamping, the last partial tile repeats
// key n-1 (its logits are masked).
template <int KB, int VB>
struct TileRegs {
    uint32_t k0[KB], k1[KB];
    uint32_t v[VB == 4 ? 8 : 2 * VB];
    float nrm;
};

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// W words from p, p aligned to ALIGN bytes, in the widest accesses that allows
// (non-temporal: the code rows are read once per launch, measured 0.329 ->
// 0.323 ms with 4-bit codes).
template <int W, int ALIGN>
__device__ __forceinline__ void load_piece(const uint8_t *p, uint32_t (&w)[W]) {
    if constexpr (ALIGN >= 16 && W % 4 == 0) {
#pragma unroll
        for (int k = 0; k < W / 4; ++k) {
            const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p) + k);
            w[4 * k] = t[0]; w[4 * k + 1] = t[1]; w[4 * k + 2] = t[2]; w[4 * k + 3] = t[3];
        }
    } else if constexpr (ALIGN >= 8 && W % 2 == 0) {
#pragma unroll
        for (int k = 0; k < W / 2; ++k) {
            const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p) + k);
            w[2 * k] = t[0]; w[2 * k + 1] = t[1];
        }
    } else {
#pragma unroll
        for (int k = 0; k < W; ++k) w[k] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p) + k);
    }
}

template <bool FULL, int KB, int VB>
__device__ __forceinline__ void load_tile(const uint8_t *kc, const uint8_t *vc, const float *kn, const float *vn,
                                          int64_t n, int64_t key0, uint32_t lane, TileRegs<KB, VB> &t) {
    constexpr uint32_t KR = 16 * KB, VR = 16 * VB;  // code bytes per key and per value row
    const uint32_t j = lane & 15u, g = lane >> 4;
    uint32_t r0 = (uint32_t)key0 + j, r1 = r0 + 16;
    uint32_t r2 = (uint32_t)key0 + (VB == 4 ? lane / 4 : lane / 2), r3 = r2 + 16;
    uint32_t rn = (uint32_t)key0 + (lane & 31u);
    if (!FULL) {
        const uint32_t last = (uint32_t)(n - 1);
        r0 = min(r0, last); r1 = min(r1, last); r2 = min(r2, last); r3 = min(r3, last); rn = min(rn, last);
    }
    constexpr int KALIGN = KB == 4 ? 16 : KB == 2 ? 8 : 4;  // of 16 KB r + 4 KB g
    load_piece<KB, KALIGN>(kc + r0 * KR + 4 * KB * g, t.k0);
    load_piece<KB, KALIGN>(kc + r1 * KR + 4 * KB * g, t.k1);
    if constexpr (VB == 4) {
        uint32_t a[4], b[4];
        load_piece<4, 16>(vc + r2 * VR + 16 * (lane % 4), a);
        load_piece<4, 16>(vc + r3 * VR + 16 * (lane % 4), b);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            t.v[k] = a[k];
            t.v[4 + k] = b[k];
        }
    } else {
        load_piece<2 * VB, VB == 2 ? 16 : 8>(vc + r2 * VR + 8 * VB * (lane % 2), t.v);
    }
    t.nrm = (lane < 32 ? kn : vn)[rn];
}

// Eight B-bit codes (bits [0, 8B) of x, the bits above zero)
// spread to one code per nibble, by halving the field groups: 4 + 4 codes to
// the two 16-bit halves, 2 + 2 to the bytes of each half, 1 + 1 to the
// nibbles of each byte.  Each step moves the upper group of every pair up by
// s bits as t + (2^s - 1) (t & M), M the upper groups' bits: the fields do not
// overlap, so the sum carries nothing.
template <int B>
__device__ __forceinline__ uint32_t spread8(uint32_t x) {
    static_assert(B == 2 || B == 3, "2- and 3-bit codes");
    if constexpr (B == 3) {
        uint32_t t = x + 15u * (x & 0x00FFF000u);   // c4..c7: bits 12-23 -> 16-27
        const uint32_t m = t & 0x0FC00FC0u;         // pairs: bits 6-11 -> 8-13 of each half
        t += (m << 1) + m;
        return t + (t & 0x38383838u);               // codes: bits 3-5 -> 4-6 of each byte
    } else {
        uint32_t t = x + 255u * (x & 0x0000FF00u);  // c4..c7: bits 8-15 -> 16-23
        t += 15u * (t & 0x00F000F0u);               // pairs: bits 4-7 -> 8-11 of each half
        return t + 3u * (t & 0x0C0C0C0Cu);          // codes: bits 2-3 -> 4-5 of each byte
    }
}

// 32 codes of B bits (an LSB-first bitstream in w[OFF .. OFF + B - 1]) as one
// code per nibble: code i at bits [4 i, 4 i + 4) of the result.
template <int B, int OFF, int N>
__device__ __forceinline__ u32x4_t widen_codes(const uint32_t (&w)[N]) {
    if constexpr (B == 4) {
        return u32x4_t{w[OFF], w[OFF + 1], w[OFF + 2], w[OFF + 3]};
    } else {
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // codes 8k .. 8k + 7: bits [8Bk, 8Bk + 8B) of the stream
            constexpr int W = 8 * B;
            const int p = W * k, wi = OFF + p / 32, sh = p % 32;
            uint32_t x = sh + W > 32 ? __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) : w[wi] >> sh;
            // the bits above the field belong to the next codes unless it ends the word
            if (sh + W != 32) x &= (1u << W) - 1u;
            o[k] = spread8<B>(x);
        }
        return u32x4_t{o[0], o[1], o[2], o[3]};
    }
}

// Per code byte, the fp16 hi and lo parts of its two levels, low nibble in
// the low half.  Entry b is a 256-byte row holding kTabCopies copies; lane l
// reads copy l % kTabCopies, so the lanes an LDS pass serves hit distinct
// banks whatever their bytes.  Two row layouts:
//   split (m > 8): the hi words (copy r at byte 4r), then the lo words (at
//     128 + 4r); the address b * 256 + 4r is one v_perm_b32 (code byte above
//     4r), the lo word the same address plus 128, each a ds_read_b32 straight
//     into an MFMA operand register;
//   paired (m <= 8): {hi, lo} of copy r at byte 8r, one ds_read_b64 per code
//     byte (half the LDS instructions: the wave's lookups were waiting to
//     issue); the level operand of a K step is {hi, lo} of two bytes.
constexpr int kTabCopies = 32;
constexpr uint32_t kTabRow = 256;  // bytes per entry

// Rows a table needs for b-bit codes widened to nibbles: bytes up to
// (2^b - 1) * 0x11.
__host__ __device__ constexpr int tab_rows(int b) { return ((1 << b) - 1) * 17 + 1; }

// The A operands for four code bytes: hi parts and lo parts, byte i in word i.
// copy4 = 4 * (lane % kTabCopies).  The reads go through volatile pointers so
// the compiler keeps them as single ds_read_b32 into the operand registers
// instead of pairing them into two-register reads that then need moves.
__device__ __forceinline__ void level_operands(const uint32_t *tb, uint32_t copy4, uint32_t w, u32x4_t &ah,
                                               u32x4_t &al) {
    typedef __attribute__((address_space(3))) const volatile uint32_t lds_word;
    const char __attribute__((address_space(3))) *base = (const char __attribute__((address_space(3))) *)tb;
    // result bytes: [0] = copy4, [1] = code byte k, [2], [3] = 0
    const uint32_t o0 = __builtin_amdgcn_perm(w, copy4, 0x0C0C0400u);
    const uint32_t o1 = __builtin_amdgcn_perm(w, copy4, 0x0C0C0500u);
    const uint32_t o2 = __builtin_amdgcn_perm(w, copy4, 0x0C0C0600u);
    const uint32_t o3 = __builtin_amdgcn_perm(w, copy4, 0x0C0C0700u);
    ah = u32x4_t{*(const lds_word *)(base + o0), *(const lds_word *)(base + o1), *(const lds_word *)(base + o2),
                 *(const lds_word *)(base + o3)};
    al = u32x4_t{*(const lds_word *)(base + o0 + 128), *(const lds_word *)(base + o1 + 128),
                 *(const lds_word *)(base + o2 + 128), *(const lds_word *)(base + o3 + 128)};
}

// Column layouts of the MFMA B operands (the 16 columns of a 16x16 tile),
// by the number of query columns QG a layout has room for:
//   QG = 16 (m <= 16): column c is query c; hi*hi + hi*lo + lo*hi go into
//     one accumulator, three MFMAs per K step.
//   QG = 8 (m <= 8): the fp16 parts go to different columns.  Column c < 8
//     holds the hi parts of query c, column 8 + c its lo parts, and the A
//     operand of a K step holds the {hi, lo} level pairs of two code bytes
//     (paired table rows), each B word twice (QueryPairs): one product leaves
//     sum (Ah + Al) Bh in column c and sum (Ah + Al) Bl in column 8 + c; their
//     sum is the result (it also carries the negligible Al Bl term).
//   QG = 4 (m <= 4): as QG = 8 for the logits (columns c and c + 4 repeat
//     query c % 4).  In the value product, bit 2 of the column is a coordinate
//     parity: column 8 * part + 4 * parity + query, so that an A row can be a
//     pair of coordinates of one key, which is one code byte as stored.
// QG = 16: hi and lo parts of the queries, one column per query.
struct QueryTriple { u32x4_t bh[4], bl[4]; };
// QG = 8, 4: the level operand of a K step holds {hi, lo} word pairs of two
// code bytes (one ds_read_b64 each), so each query word appears twice.
struct QueryPairs { u32x4_t b[8]; };
template <int QG> struct QueryOps { typedef QueryPairs type; };
template <> struct QueryOps<16> { typedef QueryTriple type; };

// {hi, lo} words of code byte k of w, from the pair-layout table (entry b,
// copy r at byte b * 256 + 8 r); copy8 = 8 * (lane % 32).
__device__ __forceinline__ uint2 level_pair(const uint32_t *tb, uint32_t copy8, uint32_t w, uint32_t sel) {
    typedef __attribute__((address_space(3))) const volatile u32x2_t lds_pair;
    const char __attribute__((address_space(3))) *base = (const char __attribute__((address_space(3))) *)tb;
    const u32x2_t v = *(const lds_pair *)(base + __builtin_amdgcn_perm(w, copy8, sel));
    return make_uint2(v.x, v.y);
}

// The value held by the lane 8 places along in the same row of 16 lanes
// (DPP row rotate by 8): the partner column of a SPLIT_N accumulator.
__device__ __forceinline__ float row_ror8(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
}

// Logits of 16 keys against the queries, pair layout (QG = 4): K step (ks, h)
// covers code bytes 2h, 2h + 1 of word ks, slots {hi, lo} of each.
__device__ __forceinline__ floatx4 key_logits_pairs(const uint32_t *tb, uint32_t copy8, u32x4_t kc,
                                                    const QueryPairs &qo) {
    floatx4 c[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint2 p0 = level_pair(tb, copy8, kc[ks], 0x0C0C0000u | ((4u + 2 * h) << 8));
            const uint2 p1 = level_pair(tb, copy8, kc[ks], 0x0C0C0000u | ((5u + 2 * h) << 8));
            c[h] = mfma1632(u32x4_t{p0.x, p0.y, p1.x, p1.y}, qo.b[2 * ks + h], c[h]);
        }
    floatx4 r = c[0] + c[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] += row_ror8(r[i]);
    return r;
}

// Logits of 16 keys (one 16-byte code piece per lane) against the queries,
// layout QG = 16 (split table, three products per K step).
__device__ __forceinline__ floatx4 key_logits_triple(const uint32_t *tb, uint32_t copy4, u32x4_t kc,
                                                     const QueryTriple &qo) {
    // two independent accumulation chains (even and odd K steps)
    floatx4 c[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        u32x4_t ah, al;
        level_operands(tb, copy4, kc[ks], ah, al);
        c[ks & 1] = mfma1632(ah, qo.bh[ks], c[ks & 1]);
        c[ks & 1] = mfma1632(ah, qo.bl[ks], c[ks & 1]);
        c[ks & 1] = mfma1632(al, qo.bh[ks], c[ks & 1]);
    }
    return c[0] + c[1];
}

// Transpose of an 8 x 8 matrix of nibbles: on entry nibble n of a[t] is
// element (t, n), on return nibble t of a[n] is.  Swaps of 4x4 blocks
// (16-bit halves), 2x2 blocks (bytes) and single nibbles.
__device__ __forceinline__ void transpose_nibbles8(uint32_t (&a)[8]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t lo = __builtin_amdgcn_perm(a[t + 4], a[t], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(a[t + 4], a[t], 0x07060302u);
        a[t] = lo;
        a[t + 4] = hi;
    }
#pragma unroll
    for (int t = 0; t < 8; t += (t % 4 == 1) ? 3 : 1) {
        const uint32_t lo = __builtin_amdgcn_perm(a[t + 2], a[t], 0x06020400u);
        const uint32_t hi = __builtin_amdgcn_perm(a[t + 2], a[t], 0x07030501u);
        a[t] = lo;
        a[t + 2] = hi;
    }
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
        const uint32_t x = a[t], y = a[t + 1];
        a[t] = (x & 0x0F0F0F0Fu) | ((y << 4) & 0xF0F0F0F0u);
        a[t + 1] = ((x >> 4) & 0x0F0F0F0Fu) | (y & 0xF0F0F0F0u);
    }
}

// Per-wave running state of the online softmax.
//   QG = 16, 8: z[n] row 4g + r <-> coordinate 32g + 8r + n.
//   QG = 4:     z[T] row 4g + r <-> coordinates 32g + 8r + 2T + parity.
template <int QG>
struct SoftmaxState {
    static constexpr int kZ = QG == 4 ? 4 : 8;
    float M, l;
    float W;             // largest weight p ||v|| seen so far, in the frame of M
    int ev;              // value scale exponent: P = p ||v|| 2^(14 - ev), 2^(ev-1) <= W < 2^ev
    floatx4 z[kZ];       // rotated value sums in the accumulator layout above
};

// Copy a tile's value codes (key r at vb + r * kVRow, one code per nibble) and
// norms into LDS.  Done before the next tile's loads are issued: waiting for
// this tile's registers then does not wait for the prefetch behind them.
template <int KB, int VB>
__device__ __forceinline__ void stage_tile(uint8_t *vb, float *nb, const TileRegs<KB, VB> &t, uint32_t lane) {
    if constexpr (VB == 4) {
        *reinterpret_cast<u32x4_t *>(vb + (lane / 4) * kVRow + 16 * (lane % 4)) =
            u32x4_t{t.v[0], t.v[1], t.v[2], t.v[3]};
        *reinterpret_cast<u32x4_t *>(vb + (16 + lane / 4) * kVRow + 16 * (lane % 4)) =
            u32x4_t{t.v[4], t.v[5], t.v[6], t.v[7]};
    } else {
        // half lane % 2 of key lane / 2: 64 codes, 32 bytes once widened
        uint8_t *row = vb + (lane / 2) * kVRow + 32 * (lane % 2);
        *reinterpret_cast<u32x4_t *>(row) = widen_codes<VB, 0>(t.v);
        *reinterpret_cast<u32x4_t *>(row + 16) = widen_codes<VB, VB>(t.v);
    }
    nb[lane] = t.nrm;
}

// Value sums of a tile, layout QG = 4.  K step i covers keys 2i and 2i + 1 of
// the lane's eight (a[2i], a[2i + 1]: 4g + t for t < 4, 16 + 4g + t - 4 after),
// slots {hi par 0, hi par 1, lo par 0, lo par 1} of each.  A for tile T, row j:
// the {hi, lo} pair of byte T of the key's code dword j, i.e. coordinates
// 8j + 2T and 8j + 2T + 1.  B: the lane's fp16 part of that key's P in the
// half of the word its parity names, the same word for the hi and lo slots.
__device__ __forceinline__ void value_sums_by_parity(const uint32_t *tb, uint32_t copy8, const uint32_t (&a)[8],
                                                     const float (&P)[8], uint2 psel, floatx4 (&z)[4]) {
    const uint2 q0 = split2(P[0], P[1]), q1 = split2(P[2], P[3]);
    const uint2 q2 = split2(P[4], P[5]), q3 = split2(P[6], P[7]);
    uint32_t bw[8];
    bw[0] = __builtin_amdgcn_perm(q0.y, q0.x, psel.x); bw[1] = __builtin_amdgcn_perm(q0.y, q0.x, psel.y);
    bw[2] = __builtin_amdgcn_perm(q1.y, q1.x, psel.x); bw[3] = __builtin_amdgcn_perm(q1.y, q1.x, psel.y);
    bw[4] = __builtin_amdgcn_perm(q2.y, q2.x, psel.x); bw[5] = __builtin_amdgcn_perm(q2.y, q2.x, psel.y);
    bw[6] = __builtin_amdgcn_perm(q3.y, q3.x, psel.x); bw[7] = __builtin_amdgcn_perm(q3.y, q3.x, psel.y);
    // key r's weight word twice: slots {hi, lo} of its level pair share it
    u32x4_t bb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) bb[i] = u32x4_t{bw[2 * i], bw[2 * i], bw[2 * i + 1], bw[2 * i + 1]};
#pragma unroll
    for (int T = 0; T < 4; ++T) {
        const uint32_t sel = 0x0C0C0000u | ((4u + T) << 8);  // [0] = copy8, [1] = byte T
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint2 p0 = level_pair(tb, copy8, a[2 * i], sel), p1 = level_pair(tb, copy8, a[2 * i + 1], sel);
            z[T] = mfma1632(u32x4_t{p0.x, p0.y, p1.x, p1.y}, bb[i], z[T]);
        }
    }
}

// Value sums of a tile, layouts QG = 8 (SPLIT_N) and 16.  B: k = 8g + t <->
// key (t < 4 ? 4g + t : 16 + 4g + t - 4) (SPLIT_N: hi parts in columns 0-7, lo
// parts in columns 8-15).  A of tile n: row j <-> coordinate 8j + n, k = 8g + t
// <-> the key above; after the transpose, byte w of word n holds coordinate
// 8j + n of keys 2w, 2w+1: one table entry each (SPLIT_N: a {hi, lo} pair, two
// bytes per K step, each weight word twice).
template <bool SPLIT_N>
__device__ __forceinline__ void value_sums_transposed(const uint32_t *tb, uint32_t copy4, uint32_t (&a)[8],
                                                      const float (&P)[8], uint32_t j, floatx4 (&z)[8]) {
    const uint2 s0 = split2(P[0], P[1]), s1 = split2(P[2], P[3]);
    const uint2 s2 = split2(P[4], P[5]), s3 = split2(P[6], P[7]);
    u32x4_t ph, pl;
    if constexpr (SPLIT_N) {
        const bool lo_col = j >= 8;
        ph = u32x4_t{lo_col ? s0.y : s0.x, lo_col ? s1.y : s1.x, lo_col ? s2.y : s2.x, lo_col ? s3.y : s3.x};
    } else {
        ph = u32x4_t{s0.x, s1.x, s2.x, s3.x};
        pl = u32x4_t{s0.y, s1.y, s2.y, s3.y};
    }
    transpose_nibbles8(a);
    if constexpr (SPLIT_N) {
        // paired table rows: bytes 0, 1 then 2, 3 of a word, {hi, lo} each; the
        // weight word of a key pair appears twice
        const u32x4_t b01 = u32x4_t{ph[0], ph[0], ph[1], ph[1]}, b23 = u32x4_t{ph[2], ph[2], ph[3], ph[3]};
        const uint32_t copy8 = 2 * copy4;
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) {
            const uint2 p0 = level_pair(tb, copy8, a[nn], 0x0C0C0400u), p1 = level_pair(tb, copy8, a[nn], 0x0C0C0500u);
            const uint2 p2 = level_pair(tb, copy8, a[nn], 0x0C0C0600u), p3 = level_pair(tb, copy8, a[nn], 0x0C0C0700u);
            z[nn] = mfma1632(u32x4_t{p0.x, p0.y, p1.x, p1.y}, b01, z[nn]);
            z[nn] = mfma1632(u32x4_t{p2.x, p2.y, p3.x, p3.y}, b23, z[nn]);
        }
    } else {
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) {
            u32x4_t ah, al;
            level_operands(tb, copy4, a[nn], ah, al);
            z[nn] = mfma1632(ah, ph, z[nn]);
            z[nn] = mfma1632(ah, pl, z[nn]);
            z[nn] = mfma1632(al, ph, z[nn]);
        }
    }
}

// One staged 32-key tile: logits on MFMA, online softmax, value sums on MFMA.
// FULL: every key of the tile is < n.  QG: the column layout (every lane of a
// column group of one query holds the same logits, maxima and weights).
// psel (QG = 4): per-lane byte selectors that place the lane's fp16 part of an
// even or odd weight of a pair in the half of the B word its parity names.
template <bool FULL, int QG>
__device__ __forceinline__ void attend_tile(const uint32_t *tbk, const uint32_t *tbv, const uint8_t *vb,
                                            const float *nb, u32x4_t k0, u32x4_t k1,
                                            const typename QueryOps<QG>::type &qo,
                                            uint2 psel, float fq, int64_t key0, int64_t n, uint32_t lane,
                                            SoftmaxState<QG> &st) {
    constexpr bool SPLIT_N = QG <= 8;
    const uint32_t j = lane & 15u, g = lane >> 4;

    // logits: rows 4g + r of tile 0 are keys 4g + r, of tile 1 keys 16 + 4g + r
    const uint32_t copy4 = 4 * (lane % kTabCopies);
    floatx4 c0, c1;
    if constexpr (SPLIT_N) {
        c0 = key_logits_pairs(tbk, 2 * copy4, k0, qo);
        c1 = key_logits_pairs(tbk, 2 * copy4, k1, qo);
    } else {
        c0 = key_logits_triple(tbk, copy4, k0, qo);
        c1 = key_logits_triple(tbk, copy4, k1, qo);
    }
    const float4 kn0 = *reinterpret_cast<const float4 *>(nb + 4 * g);
    const float4 kn1 = *reinterpret_cast<const float4 *>(nb + 16 + 4 * g);
    const float4 vn0 = *reinterpret_cast<const float4 *>(nb + 32 + 4 * g);
    const float4 vn1 = *reinterpret_cast<const float4 *>(nb + 48 + 4 * g);
    const float knr[8] = {kn0.x, kn0.y, kn0.z, kn0.w, kn1.x, kn1.y, kn1.z, kn1.w};
    const float vnr[8] = {vn0.x, vn0.y, vn0.z, vn0.w, vn1.x, vn1.y, vn1.z, vn1.w};
    float s[8], vr[8], smax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const float cv = r < 4 ? c0[r] : c1[r - 4];
        s[r] = cv * knr[r] * fq;
        vr[r] = vnr[r];
        if (!FULL) {
            const bool live = key0 + (r < 4 ? 4 * g + r : 16 + 4 * g + (r - 4)) < n;
            s[r] = live ? s[r] : -INFINITY;
            vr[r] = live ? vr[r] : 0.0f;
        }
        smax = fmaxf(smax, s[r]);
    }
    smax = max_over_rows(smax);
    const float Mn = fmaxf(st.M, smax);
    const float alpha = __builtin_amdgcn_exp2f(st.M - Mn);
    // weights w = p ||v||; the fp16 scale of the value operand follows the
    // largest weight of the chunk so far (not the largest norm: a key of huge
    // norm and negligible weight must not push the others below fp16 range)
    float w[8], wmax = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const float pr = __builtin_amdgcn_exp2f(s[r] - Mn);
        st.l = r == 0 ? st.l * alpha + pr : st.l + pr;
        w[r] = pr * vr[r];
        wmax = fmaxf(wmax, w[r]);
    }
    wmax = max_over_rows(wmax);
    const float Wn = fmaxf(st.W * alpha, wmax);
    const int evn = Wn > 0.0f ? exponent_above(Wn) : st.ev;
    // rescale the running sums to the new max and value scale (skipped when
    // neither moved for any query of the wave)
    const float rz = __builtin_amdgcn_ldexpf(alpha, st.ev - evn);
    st.M = Mn;
    st.W = Wn;
    st.ev = evn;
    if (__any(rz != 1.0f)) {
#pragma unroll
        for (int nn = 0; nn < SoftmaxState<QG>::kZ; ++nn) st.z[nn] *= rz;
    }
    float P[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) P[r] = __builtin_amdgcn_ldexpf(w[r], 14 - evn);
    // value codes: word tt = code dword j (coordinates 8j .. 8j+7) of key
    // (tt < 4 ? 4g + tt : 16 + 4g + tt - 4), the keys of this lane's P values
    uint32_t a[8];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
        const uint32_t key = tt < 4 ? 4 * g + tt : 16 + 4 * g + (tt - 4);
        a[tt] = *reinterpret_cast<const uint32_t *>(vb + key * kVRow + 4 * j);
    }
    if constexpr (QG == 4)
        value_sums_by_parity(tbv, 2 * copy4, a, P, psel, st.z);
    else
        value_sums_transposed<SPLIT_N>(tbv, copy4, a, P, j, st.z);
}

template <int QG, int KB, int VB>
__global__ __launch_bounds__(kABlock) void k_attn_partial(const AttnArgs a) {
    constexpr bool SPLIT_N = QG <= 8;
    constexpr bool SHARED = KB == VB;  // one codebook, one table
    constexpr uint32_t WK = tab_rows(KB) * kTabRow / 4, WV = tab_rows(VB) * kTabRow / 4;  // table words
    __shared__ __attribute__((aligned(16))) uint32_t tabs[WK + (SHARED ? 0 : WV)];
    __shared__ __attribute__((aligned(16))) uint8_t vbuf[kAWaves][32 * kVRow];
    __shared__ __attribute__((aligned(16))) float nbuf[kAWaves][64];
    for (uint32_t k = threadIdx.x; k < WK + (SHARED ? 0 : WV); k += kABlock) {
        const bool vtab = k >= WK;
        const uint32_t kk = vtab ? k - WK : k;
        const uint32_t v = kk / (kTabRow / 4), r = kk % (kTabRow / 4);
        const float *lev = vtab ? a.lev_v : a.lev_k;
        const uint2 e = split2(lev[v & 15u], lev[v >> 4]);
        tabs[k] = SPLIT_N ? ((r & 1u) ? e.y : e.x) : (r < kTabCopies ? e.x : e.y);
    }
    __syncthreads();
    const uint32_t *tbk = tabs, *tbv = SHARED ? tabs : tabs + WK;

    const uint32_t lane = lane_id(), j = lane & 15u, g = lane >> 4;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t gw = (int64_t)blockIdx.x * kAWaves + wave;
    if (gw >= a.heads * a.chunks) return;  // whole wave; no block barrier follows
    const int64_t head = gw / a.chunks;
    const int chunk = (int)(gw % a.chunks);
    const int64_t n = a.n;
    const int64_t tiles = (n + 31) / 32;
    const int64_t t_begin = tiles * chunk / a.chunks, t_end = tiles * (chunk + 1) / a.chunks;

    // --- queries: q~ = H D_k q, scaled by 2^(14 - e) into fp16 range.  The
    // B operand of the logits for lane (query j, group g), K step ks, word w is
    // the coordinate pair 32g + 8ks + 2w (+1), held by lane 16g + 4ks + w after
    // the transform; every lane fetches it for every query and keeps query j's.
    float qscale_mine = 1.0f;  // power of two applied to query j
    float qp[4][4][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int w = 0; w < 4; ++w) qp[ks][w][0] = qp[ks][w][1] = 0.0f;
    // one query's rotation, scaling and hand-out of its operand words
    auto rotate_query = [&](int i) {
        const int iq = i < a.m ? i : a.m - 1;
        const float2 qv = reinterpret_cast<const float2 *>(a.q + (head * a.m + iq) * kAD)[lane];
        const uint32_t sb = a.dsign_k[lane >> 4] >> ((2 * lane) & 31);
        float v0 = (sb & 1u) ? -qv.x : qv.x;
        float v1 = (sb & 2u) ? -qv.y : qv.y;
        fwht128_pairs(v0, v1, lane);
        const float mx = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
        const float sc = mx > 0.0f ? pow2i(min(14 - exponent_above(mx), 126)) : 1.0f;
        v0 *= sc;
        v1 *= sc;
        const bool mine = i < a.m && (uint32_t)i == j % (uint32_t)QG;
        if (mine) qscale_mine = sc;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int src = 16 * (int)g + 4 * ks + w;
                const float p0 = __shfl(v0, src), p1 = __shfl(v1, src);
                qp[ks][w][0] = mine ? p0 : qp[ks][w][0];
                qp[ks][w][1] = mine ? p1 : qp[ks][w][1];
            }
    };
    if constexpr (QG == 4) {
        // the four rotations unrolled (queries past m repeat the last one and
        // are selected by no lane), so their shuffle chains overlap; with more
        // queries the unrolled chains would not fit the registers
#pragma unroll
        for (int i = 0; i < QG; ++i) rotate_query(i);
    } else {
        for (int i = 0; i < a.m; ++i) rotate_query(i);
    }
    typename QueryOps<QG>::type qo;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        uint32_t h[4], l[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint2 sp = split2(qp[ks][w][0], qp[ks][w][1]);
            h[w] = sp.x;
            l[w] = sp.y;
        }
        if constexpr (SPLIT_N) {
            const bool lo_col = j >= 8;
            const uint32_t b0 = lo_col ? l[0] : h[0], b1 = lo_col ? l[1] : h[1];
            const uint32_t b2 = lo_col ? l[2] : h[2], b3 = lo_col ? l[3] : h[3];
            qo.b[2 * ks] = u32x4_t{b0, b0, b1, b1};
            qo.b[2 * ks + 1] = u32x4_t{b2, b2, b3, b3};
        } else {
            qo.bh[ks] = u32x4_t{h[0], h[1], h[2], h[3]};
            qo.bl[ks] = u32x4_t{l[0], l[1], l[2], l[3]};
        }
    }
    // logits in base-2 units: s = C * ||k|| * fq
    const float fq = a.scale * 1.4426950408889634f / ((float)kAD * qscale_mine);

    const uint8_t *kc = a.kc + head * n * (16 * KB);
    const uint8_t *vc = a.vc + head * n * (16 * VB);
    const float *kn = a.kn + head * n;
    const float *vn = a.vn + head * n;
    uint8_t *vb = vbuf[wave];
    float *nb = nbuf[wave];

    SoftmaxState<QG> st;
    st.M = -INFINITY;
    st.l = 0.0f;
    st.W = 0.0f;
    st.ev = 0;
#pragma unroll
    for (int nn = 0; nn < SoftmaxState<QG>::kZ; ++nn) st.z[nn] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    // QG = 4: byte selectors of this lane's B words (bytes 0-3 of the perm
    // source are the hi pair, 4-7 the lo pair; an even weight is the low half)
    uint2 psel = make_uint2(0u, 0u);
    if constexpr (QG == 4) {
        const uint32_t b = j >= 8 ? 4u : 0u, par = (j >> 2) & 1u;
        const uint32_t ev16 = b | ((b + 1) << 8), od16 = (b + 2) | ((b + 3) << 8);
        psel.x = par ? (ev16 << 16) | 0x0C0Cu : 0x0C0C0000u | ev16;
        psel.y = par ? (od16 << 16) | 0x0C0Cu : 0x0C0C0000u | od16;
    }

    // full tiles with the next one's loads in flight (two register sets), then
    // the partial last tile if n is not a multiple of 32
    const int64_t t_full = min(t_end, n / 32);
    TileRegs<KB, VB> ra, rb;
    int64_t tile = t_begin;
    if (tile < t_full) load_tile<true>(kc, vc, kn, vn, n, tile * 32, lane, ra);
    while (tile < t_full) {
        stage_tile(vb, nb, ra, lane);
        if (tile + 1 < t_full) load_tile<true>(kc, vc, kn, vn, n, (tile + 1) * 32, lane, rb);
        attend_tile<true, QG>(tbk, tbv, vb, nb, widen_codes<KB, 0>(ra.k0), widen_codes<KB, 0>(ra.k1), qo, psel,
                              fq, tile * 32, n, lane, st);
        if (++tile >= t_full) break;
        stage_tile(vb, nb, rb, lane);
        if (tile + 1 < t_full) load_tile<true>(kc, vc, kn, vn, n, (tile + 1) * 32, lane, ra);
        attend_tile<true, QG>(tbk, tbv, vb, nb, widen_codes<KB, 0>(rb.k0), widen_codes<KB, 0>(rb.k1), qo, psel,
                              fq, tile * 32, n, lane, st);
        ++tile;
    }
    if (t_full < t_end) {
        load_tile<false>(kc, vc, kn, vn, n, t_full * 32, lane, ra);
        stage_tile(vb, nb, ra, lane);
        attend_tile<false, QG>(tbk, tbv, vb, nb, widen_codes<KB, 0>(ra.k0), widen_codes<KB, 0>(ra.k1), qo, psel,
                               fq, t_full * 32, n, lane, st);
    }

    // SPLIT_N: column j + 8 holds the lo-part sums of column j (DPP, all lanes)
    if constexpr (SPLIT_N) {
#pragma unroll
        for (int nn = 0; nn < SoftmaxState<QG>::kZ; ++nn)
#pragma unroll
            for (int r = 0; r < 4; ++r) st.z[nn][r] += row_ror8(st.z[nn][r]);
    }
    // l: each lane group g summed its own keys
    float l = st.l;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if constexpr (QG == 4) {
        // lane (column j < 8): query j % 4, coordinates of parity j / 4
        const uint32_t qi = j & 3u, par = j >> 2;
        if (j < 8 && (int)qi < a.m) {
            float *rec = a.ws + ((head * a.chunks + chunk) * a.m + qi) * kAttnRecord;
            const float zs = __builtin_amdgcn_ldexpf(1.0f / (float)kAD, st.ev - 14);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int T = 0; T < 4; ++T) rec[32 * g + 8 * r + 2 * T + par] = st.z[T][r] * zs;
            if (g == 0 && par == 0) {
                rec[kAD] = st.M;
                rec[kAD + 1] = l;
            }
        }
    } else if ((int)j < a.m) {
        float *rec = a.ws + ((head * a.chunks + chunk) * a.m + j) * kAttnRecord;
        // accumulator row 4g + r of tile n is coordinate 32g + 8r + n
        const float zs = __builtin_amdgcn_ldexpf(1.0f / (float)kAD, st.ev - 14);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float4 lo, hi;
            lo.x = st.z[0][r] * zs; lo.y = st.z[1][r] * zs; lo.z = st.z[2][r] * zs; lo.w = st.z[3][r] * zs;
            hi.x = st.z[4][r] * zs; hi.y = st.z[5][r] * zs; hi.z = st.z[6][r] * zs; hi.w = st.z[7][r] * zs;
            reinterpret_cast<float4 *>(rec + 32 * g + 8 * r)[0] = lo;
            reinterpret_cast<float4 *>(rec + 32 * g + 8 * r)[1] = hi;
        }
        if (g == 0) {
            rec[kAD] = st.M;
            rec[kAD + 1] = l;
        }
    }
}

// Merge a head's partial records for one query and apply D_v H:
// out = D_v H (sum_c 2^(M_c - M) z_c) / (sum_c 2^(M_c - M) l_c).
__global__ __launch_bounds__(kBlock) void k_attn_combine(const AttnArgs a) {
    const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t qi = (int64_t)blockIdx.x * kWaves + wave;
    if (qi >= a.heads * a.m) return;
    const int64_t head = qi / a.m;
    const int i = (int)(qi % a.m);
    const float *rec0 = a.ws + (head * a.chunks * a.m + i) * kAttnRecord;
    const int64_t step = (int64_t)a.m * kAttnRecord;
    // chunk maxima and weighted sums, one chunk per lane (the loads of all
    // chunks are in flight together instead of one round trip per chunk)
    float M = -INFINITY;
    for (int c = (int)lane; c < a.chunks; c += 64) M = fmaxf(M, rec0[c * step + kAD]);
    M = wave_max(M);
    float l = 0.0f;
    for (int c = (int)lane; c < a.chunks; c += 64)
        l = fmaf(__builtin_amdgcn_exp2f(rec0[c * step + kAD] - M), rec0[c * step + kAD + 1], l);
    l = wave_sum(l);
    float z0 = 0.0f, z1 = 0.0f;
#pragma unroll 4
    for (int c = 0; c < a.chunks; ++c) {
        const float *rec = rec0 + c * step;
        const float w = __builtin_amdgcn_exp2f(rec[kAD] - M);
        const float2 zv = reinterpret_cast<const float2 *>(rec)[lane];
        z0 = fmaf(w, zv.x, z0);
        z1 = fmaf(w, zv.y, z1);
    }
    const float inv = 1.0f / l;
    z0 *= inv;
    z1 *= inv;
    fwht128_pairs(z0, z1, lane);
    const uint32_t sb = a.dsign_v[lane >> 4] >> ((2 * lane) & 31);
    float2 o;
    o.x = (sb & 1u) ? -z0 : z0;
    o.y = (sb & 2u) ? -z1 : z1;
    reinterpret_cast<float2 *>(a.out + (head * a.m + i) * kAD)[lane] = o;
}

}  // namespace

namespace {

// The partial kernel for the queries per head (one of three operand layouts).
template <int KB, int VB>
hipError_t launch_partial(const AttnArgs &a, dim3 grid, hipStream_t s) {
    if (a.m <= 4) return launch(k_attn_partial<4, KB, VB>, grid, dim3(kABlock), s, a);
    if (a.m <= 8) return launch(k_attn_partial<8, KB, VB>, grid, dim3(kABlock), s, a);
    return launch(k_attn_partial<16, KB, VB>, grid, dim3(kABlock), s, a);
}

}  // namespace

hipError_t attention_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            // with device `dev` current: this device's copy of the array
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_attention(const AttnArgs &a, hipStream_t s) {
    const int64_t waves = a.heads * a.chunks;
    const dim3 grid((unsigned)((waves + kAWaves - 1) / kAWaves));
    hipError_t e = hipErrorInvalidValue;
    switch (a.kbits * 8 + a.vbits) {
    case 4 * 8 + 4: e = launch_partial<4, 4>(a, grid, s); break;
    case 4 * 8 + 3: e = launch_partial<4, 3>(a, grid, s); break;
    case 4 * 8 + 2: e = launch_partial<4, 2>(a, grid, s); break;
    case 3 * 8 + 4: e = launch_partial<3, 4>(a, grid, s); break;
    case 3 * 8 + 3: e = launch_partial<3, 3>(a, grid, s); break;
    case 3 * 8 + 2: e = launch_partial<3, 2>(a, grid, s); break;
    case 2 * 8 + 4: e = launch_partial<2, 4>(a, grid, s); break;
    case 2 * 8 + 3: e = launch_partial<2, 3>(a, grid, s); break;
    case 2 * 8 + 2: e = launch_partial<2, 2>(a, grid, s); break;
    }
    if (e != hipSuccess) return e;
    const int64_t rows = a.heads * a.m;
    return launch(k_attn_combine, dim3((unsigned)((rows + kWaves - 1) / kWaves)), dim3(kBlock), s, a);
}

}  // namespace rht
