// rht_kv128.hip -- the d = 128, fp16, 4-bit encoder and decoder with the
// H_32 factor of the transform on MFMA (KV-cache head vectors).
//
// Method: web page "Random-rotation quantization" (brain.bigb.es): rotate each
// vector by Pi = H D / sqrt(d) ("Why rotation works"), quantize every rotated
// coordinate with the N(0,1) Lloyd-Max codebook ("History", EDEN item), decode
// with Pi^T ("intro", step 3).
#include "rht_device.h"

namespace rht {
namespace {

// ---------------------------------------------------------------------------
// Hadamard-as-GEMM variant for d = 128 (fp16 data, 4-bit codes).
//
// H_128 = H_4 (x) H_32 over the coordinate split e = 32 a + b (Sylvester
// entries (-1)^popcount(e & e') factor over the two bit groups).  The H_32
// factor runs on v_mfma_f32_32x32x16_f16; the H_4 factor is two butterfly
// stages.  Encoder: the 32 vectors of a wave's tile are the N dimension; lane
// l serves vector j = l % 32 with half h = l / 32, and in the K step (a', kk)
// it supplies coordinates 32 a' + 16 h + 8 kk + t, t = 0..7 (16 bytes of
// fp16).  Decoder: the N dimension is 16 vectors x 2 coordinate blocks (see
// dequantize_tile).
// Output row i of a 32x32 tile is mapped to b = pi(i) so that the lane holds
// b = 16 h + r in accumulator register r: the lane ends up with 16
// consecutive coordinates per block a, i.e. whole 64-bit code words.
// Products of fp16 values and +-1 are exact; accumulation is fp32.

// b = pi(i) for the accumulator row i = 8 (r / 4) + 4 h + r % 4  ->  16 h + r.
__device__ __forceinline__ uint32_t acc_row_to_b(uint32_t i) {
    return 16u * ((i >> 2) & 1u) + 4u * (i >> 3) + (i & 3u);
}

__device__ __forceinline__ floatx16 mfma16(u32x4_t a, u32x4_t b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

// Operand A for K step kk: A[i][k] = H_32[pi(i)][16 (k / 8) + 8 kk + k % 8], times
// the sign s_{32 a' + that coordinate} when `dsign` is given.
__device__ __forceinline__ u32x4_t hadamard_operand(uint32_t lane, int ap, int kk, const uint32_t *dsign) {
    const uint32_t pb = acc_row_to_b(lane & 31u), h = lane >> 5;
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
        uint32_t half2 = 0;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t b = 16u * h + 8u * kk + t + u;
            uint32_t neg = __builtin_popcount(pb & b) & 1u;
            if (dsign) {
                const uint32_t e = 32u * ap + b;
                neg ^= (dsign[e >> 5] >> (e & 31)) & 1u;
            }
            half2 |= (neg ? 0xBC00u : 0x3C00u) << (16 * u);
        }
        w[t / 2] = half2;
    }
    return u32x4_t{w[0], w[1], w[2], w[3]};
}

// Operand A for the decoder's K step m, whose K slots carry the fp16 hi and lo
// parts of four coordinates: slot t of half h is coordinate 16 h + 4 m +
// {0,1,0,1,2,3,2,3}[t] (hi parts in t = 0,1,4,5, lo parts in t = 2,3,6,7).
__device__ __forceinline__ u32x4_t hadamard_operand_hilo(uint32_t lane, int m) {
    const uint32_t pb = acc_row_to_b(lane & 31u), h = lane >> 5;
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
        uint32_t half2 = 0;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tt = t + u;
            const uint32_t b = 16u * h + 4u * m + (uint32_t)((tt & 1) + 2 * (tt >> 2));
            half2 |= ((__builtin_popcount(pb & b) & 1u) ? 0xBC00u : 0x3C00u) << (16 * u);
        }
        w[t / 2] = half2;
    }
    return u32x4_t{w[0], w[1], w[2], w[3]};
}

// H_4 across the four accumulators, in place: c[a] <- sum_a' (-1)^popcount(a & a') c[a'].
__device__ __forceinline__ void hadamard4(floatx16 (&c)[4]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float u0 = c[0][r] + c[1][r], u1 = c[0][r] - c[1][r];
        const float u2 = c[2][r] + c[3][r], u3 = c[2][r] - c[3][r];
        c[0][r] = u0 + u2;
        c[2][r] = u0 - u2;
        c[1][r] = u1 + u3;
        c[3][r] = u1 - u3;
    }
}

// LDS staging for the d = 128 MFMA kernels.  A wave works on a tile of 32
// rows (encoder) or 16 rows (decoder).  Global traffic is coalesced: each
// load/store instruction of a wave moves one contiguous KiB (four 256-byte
// fp16 rows, or sixteen 64-byte code rows).  Inside LDS, the 16-byte chunk c of tile row r sits at chunk position
// c ^ (r mod 16) (fp16 rows) or c ^ (r mod 4) (code rows), so the per-lane
// reads and writes of the MFMA layout (one row per lane) hit distinct banks.
typedef __attribute__((address_space(3))) void lds_void;

// Streaming accesses.  Every byte these kernels move is touched once, so the
// fp16 rows are copied in and the code rows and fp16 output are stored with
// the non-temporal cache policy.  With ordinary stores a launch leaves up to
// the caches' worth of dirty lines behind, and the launch after it (the next
// tensor, the other direction) pays for their write-back: measured in the
// quantize K, quantize V, dequantize K, dequantize V sequence, the step took
// 2.15 ms with ordinary accesses and 2.01-2.02 ms with these (the encoder
// itself 0.53-0.57 -> 0.49 ms).  The decoder's code copies keep the default
// policy: making them non-temporal as well slowed the decoder.
constexpr int kStreamCopy = 2;  // cache-policy bits of global_load_lds: nt
__device__ __forceinline__ void stream_store(uint4 v, void *p) {
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, static_cast<u32x4_t *>(p));
}

// Wait until this wave's direct global -> LDS copies have landed.  The compiler
// does not reliably order such copies against later LDS reads of the same
// buffer, so every read of a staged tile is preceded by this wait (the
// "memory" clobber keeps memory accesses from moving across it).
__device__ __forceinline__ void wait_lds_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

constexpr int kRowsPerWave = 32;
constexpr int kTileBytes = kRowsPerWave * 256;   // fp16 rows of one wave
constexpr int kCodeTileBytes = kRowsPerWave * 64;

__device__ __forceinline__ uint32_t x_chunk(uint32_t r, uint32_t c) { return 16u * r + (c ^ (r & 15u)); }
__device__ __forceinline__ uint32_t c_chunk(uint32_t r, uint32_t c) { return 4u * r + (c ^ (r & 3u)); }

// Direct global -> LDS copy of the 32 fp16 rows starting at row0 (rows past
// the end repeat the last row).  Instruction k fills LDS chunks 64k .. 64k+63.
__device__ __forceinline__ void stage_rows(const uint16_t *x, int64_t row0, int64_t n, char *lds_tile,
                                           uint32_t lane) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t r = 4u * k + (lane >> 4), pos = lane & 15u;
        const int64_t row = row0 + r < n ? row0 + r : n - 1;
        const uint4 *src = reinterpret_cast<const uint4 *>(x + row * 128) + (pos ^ (r & 15u));
        __builtin_amdgcn_global_load_lds(src, (lds_void *)(lds_tile + 1024 * k), 16, 0, kStreamCopy);
    }
}

// One tile of the encoder: read the staged rows from `tile`, transform,
// quantize, write codes and norms.  `next` is the other staging buffer; the
// following tile's rows are copied into it while this one is processed.
__device__ __forceinline__ void quantize_tile128(const QuantArgs &a, const uint2 *lut, const u32x4_t (&A)[4][2],
                                                 const char *tile, char *next, char *ct, int64_t v0,
                                                 int64_t v0_next, uint32_t lane) {
    constexpr int D = 128;
    const uint32_t j = lane & 31u, h = lane >> 5;
    u32x4_t raw[4][2];
    wait_lds_copies();
#pragma unroll
    for (int ap = 0; ap < 4; ++ap)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            raw[ap][kk] = *reinterpret_cast<const u32x4_t *>(tile + 16 * x_chunk(j, 4 * ap + 2 * h + kk));
    stage_rows(static_cast<const uint16_t *>(a.x), v0_next, a.n, next, lane);
    float ss = 0.0f, ss2 = 0.0f;
    floatx16 c[4];
#pragma unroll
    for (int ap = 0; ap < 4; ++ap) {
        c[ap] = floatx16{};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            c[ap] = mfma16(A[ap][kk], raw[ap][kk], c[ap]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q & 1)
                    ss2 = dot2(raw[ap][kk][q], raw[ap][kk][q], ss2);
                else
                    ss = dot2(raw[ap][kk][q], raw[ap][kk][q], ss);
            }
        }
    }
    ss += ss2;
    ss += __shfl_xor(ss, 32);
    const float nrm = sqrtf(ss);
    const float inv16 = ss > 0.0f ? 16.0f / nrm : 0.0f;
    hadamard4(c);
#pragma unroll
    for (int ap = 0; ap < 4; ++ap) {
        uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
        for (int r = 0; r < 8; ++r) w0 |= nearest_code<D>(lut, c[ap][r] * inv16) << (4 * r);
#pragma unroll
        for (int r = 0; r < 8; ++r) w1 |= nearest_code<D>(lut, c[ap][r + 8] * inv16) << (4 * r);
        // code bytes 16 ap + 8 h .. +8 of row j: half of 16-byte chunk ap
        *reinterpret_cast<uint2 *>(ct + 16 * c_chunk(j, ap) + 8 * h) = make_uint2(w0, w1);
    }
    const int64_t vec = v0 + j;
    if (h == 0 && vec < a.n) a.scale[vec] = nrm;
    // coalesced code stores: instruction k covers tile rows 16k .. 16k+15
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t r = 16u * k + (lane >> 2), cc = lane & 3u;
        const uint4 val = *reinterpret_cast<const uint4 *>(ct + 16 * c_chunk(r, cc));
        if (v0 + r < a.n) stream_store(val, reinterpret_cast<uint4 *>(a.codes + (v0 + r) * 64) + cc);
    }
}

__global__ __launch_bounds__(kBlock) void k_quantize_mfma128(const QuantArgs a) {
    constexpr int D = 128, VPB = kWaves * kRowsPerWave;
    __shared__ uint2 lut[Lut<D>::kCells];
    // two staging buffers as separate objects so the compiler can tell the
    // copy into one from the reads of the other
    __shared__ __attribute__((aligned(16))) char xbuf0[kWaves][kTileBytes];
    __shared__ __attribute__((aligned(16))) char xbuf1[kWaves][kTileBytes];
    __shared__ __attribute__((aligned(16))) char cbuf[kWaves][kCodeTileBytes];
    build_lut<Lut<D>::kCells, Lut<D>::kOff>(lut, a.thr, 15);
    __syncthreads();

    const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
    u32x4_t A[4][2];
#pragma unroll
    for (int ap = 0; ap < 4; ++ap)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) A[ap][kk] = hadamard_operand(lane, ap, kk, a.dsign);

    const int64_t stride = (int64_t)gridDim.x * VPB;
    const int64_t first = (int64_t)blockIdx.x * VPB + wave * kRowsPerWave;
    const int64_t limit = a.n + wave * kRowsPerWave;  // a block iteration runs while its first row < n
    stage_rows(static_cast<const uint16_t *>(a.x), first, a.n, xbuf0[wave], lane);
    for (int64_t v0 = first; v0 < limit; v0 += 2 * stride) {
        quantize_tile128(a, lut, A, xbuf0[wave], xbuf1[wave], cbuf[wave], v0, v0 + stride, lane);
        if (v0 + stride >= limit) break;
        quantize_tile128(a, lut, A, xbuf1[wave], xbuf0[wave], cbuf[wave], v0 + stride, v0 + 2 * stride, lane);
    }
}

// The decoder works on tiles of 16 rows: trivial kernels that stream the
// decode shape (68 bytes in, 256 out per row) through LDS ran 0.4815 ms per
// 2^23 rows in 16-row wave steps against 0.497 ms in 32-row steps.  The 32
// columns of the 32 x 32 product are then 16 rows x 2 of the four 32-coordinate
// blocks: column n = 16 p + j is row j, and accumulator q holds block 2 q + p
// (the H_32 operand is the same for every block).
constexpr int kDecRows = 16;
constexpr int kDecScaleOff = kDecRows * 64;        // code rows: 1 KiB
constexpr int kDecTileBytes = kDecScaleOff + 256;  // scales: 4 bytes per lane, rows repeating
constexpr int kDecOutBytes = kDecRows * 256;

// Direct global -> LDS copy of the 16 code rows at row0 (one KiB: chunk c of
// row r at position c_chunk(r, c)) and their scales (bytes kDecScaleOff + 4 l,
// lane l taking row l % 16).  Rows past the end repeat the last row.
__device__ __forceinline__ void stage_codes(const DequantArgs &a, int64_t row0, char *tile, uint32_t lane) {
    const uint32_t r = lane >> 2, pos = lane & 3u;
    const int64_t row = row0 + r < a.n ? row0 + r : a.n - 1;
    const uint4 *src = reinterpret_cast<const uint4 *>(a.codes + row * 64) + (pos ^ (r & 3u));
    __builtin_amdgcn_global_load_lds(src, (lds_void *)tile, 16, 0, 0);
    const int64_t srow = row0 + (lane & 15u) < a.n ? row0 + (lane & 15u) : a.n - 1;
    __builtin_amdgcn_global_load_lds(a.scale + srow, (lds_void *)(tile + kDecScaleOff), 4, 0, 0);
}

// One tile of the decoder: codes from the staged `tile`, the next tile's codes
// copied into `next` meanwhile, output transposed through `yt` into coalesced
// stores.  WHOLE: this tile and the wave's previous one have all 16 rows below
// n.  The previous tile then issued all four of its stores after this tile's
// copies (codes and scales), so waiting until at most four memory operations are
// outstanding covers the copies and leaves the stores in flight (vmcnt counts
// loads and stores together and retires them in order).  The staged code reads
// sit in the same asm block as that wait: the compiler would otherwise put a
// full wait in front of ordinary LDS reads that follow direct copies.  Its
// outputs are early-clobber: no read's data register may be an address register
// of a later read in the block.  This tile's stores need no row check.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const char lds_cchar;
template <bool WHOLE>
__device__ __forceinline__ void dequantize_tile(const DequantArgs &a, const uint2 *tab, const u32x4_t (&A)[4],
                                                const uint32_t (&om)[2][8], const char *tile, char *next, char *yt,
                                                int64_t v0, int64_t v0_next, uint32_t lane) {
    constexpr int D = 128;
    const uint32_t j = lane & 15u, p = (lane >> 4) & 1u, h = lane >> 5;
    uint2 cw[2];  // code bytes 16 (2 q + p) + 8 h .. +8 of row j
    float scale;
    if constexpr (WHOLE) {
        const uint32_t base = (uint32_t)(uintptr_t)(lds_cchar *)tile;  // LDS byte address
        u32x2_t r0, r1;
        asm volatile("s_waitcnt vmcnt(4)\n\t"
                     "ds_read_b64 %0, %3\n\t"
                     "ds_read_b64 %1, %4\n\t"
                     "ds_read_b32 %2, %5\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(r0), "=&v"(r1), "=&v"(scale)
                     : "v"(base + 16 * c_chunk(j, p) + 8 * h), "v"(base + 16 * c_chunk(j, 2 + p) + 8 * h),
                       "v"(base + kDecScaleOff + 4 * j)
                     : "memory");
        cw[0] = make_uint2(r0.x, r0.y);
        cw[1] = make_uint2(r1.x, r1.y);
    } else {
        wait_lds_copies();
#pragma unroll
        for (int q = 0; q < 2; ++q)
            cw[q] = *reinterpret_cast<const uint2 *>(tile + 16 * c_chunk(j, 2 * q + p) + 8 * h);
        scale = *reinterpret_cast<const float *>(tile + kDecScaleOff + 4 * j);
    }
    const float alpha = scale * (1.0f / D);
    // the next tile's codes and scales load into LDS during this one
    stage_codes(a, v0_next, next, lane);
    floatx16 c[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        c[q] = floatx16{};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            // code bytes 2m, 2m+1 of the lane's eight: coordinates 16 h + 4m .. +3 of block 2 q + p
            const uint32_t wd = m < 2 ? cw[q].x : cw[q].y;
            const uint2 e0 = tab[(wd >> (16 * (m & 1))) & 0xFFu];
            const uint2 e1 = tab[(wd >> (16 * (m & 1) + 8)) & 0xFFu];
            c[q] = mfma16(A[m], u32x4_t{e0.x, e0.y, e1.x, e1.y}, c[q]);
        }
    }
    // H_4 over the blocks a = 2 q + p: the butterfly over q in the lane, then the
    // one over p, after a swap with lane l ^ 16 (same row, other p) leaves lane p
    // with both p-values of q = p; the lane then holds blocks 2 p and 2 p + 1.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float d0 = c[0][r] + c[1][r], d1 = c[0][r] - c[1][r];
        const auto sw = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, d0),
                                                         __builtin_bit_cast(uint32_t, d1), false, false);
        const uint32_t sx = sw[0], sy = sw[1];
        const float x = __builtin_bit_cast(float, sx), y = __builtin_bit_cast(float, sy);
        c[0][r] = x + y;
        c[1][r] = x - y;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        uint32_t o[8];
#pragma unroll
        for (int pr = 0; pr < 8; ++pr) {
            const _Float16 lo = (_Float16)(c[s][2 * pr] * alpha);
            const _Float16 hi = (_Float16)(c[s][2 * pr + 1] * alpha);
            o[pr] = ((uint32_t)__builtin_bit_cast(uint16_t, lo) |
                     ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16)) ^ om[s][pr];
        }
        // fp16 bytes 64 (2 p + s) + 32 h .. +32 of row j: chunks 4 (2 p + s) + 2 h, +1
        const uint32_t ch = 4u * (2u * p + s) + 2u * h;
        *reinterpret_cast<uint4 *>(yt + 16 * x_chunk(j, ch)) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4 *>(yt + 16 * x_chunk(j, ch + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
    }
    // coalesced stores: instruction k covers tile rows 4k .. 4k+3
    uint16_t *y = static_cast<uint16_t *>(a.y);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t r = 4u * k + (lane >> 4), cc = lane & 15u;
        const uint4 val = *reinterpret_cast<const uint4 *>(yt + 16 * x_chunk(r, cc));
        if (WHOLE || v0 + r < a.n) stream_store(val, reinterpret_cast<uint4 *>(y + (v0 + r) * D) + cc);
    }
}

__global__ __launch_bounds__(kBlock) void k_dequantize_mfma128(const DequantArgs a) {
    constexpr int VPB = kWaves * kDecRows;
    // per code byte: (hi parts, lo parts) of its two levels as packed fp16
    __shared__ uint2 tab[256];
    __shared__ __attribute__((aligned(16))) char cbuf0[kWaves][kDecTileBytes];
    __shared__ __attribute__((aligned(16))) char cbuf1[kWaves][kDecTileBytes];
    __shared__ __attribute__((aligned(16))) char ybuf[kWaves][kDecOutBytes];
    {
        const uint32_t v = threadIdx.x;
        const float c0 = a.lev[v & 15u], c1 = a.lev[v >> 4];
        const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
        const _Float16 l0 = (_Float16)(c0 - (float)h0), l1 = (_Float16)(c1 - (float)h1);
        tab[v] = make_uint2((uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16),
                            (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16));
    }
    __syncthreads();

    const uint32_t lane = lane_id(), p = (lane >> 4) & 1u, h = lane >> 5, wave = threadIdx.x >> 6;
    u32x4_t A[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) A[m] = hadamard_operand_hilo(lane, m);
    // D applied to the output: packed fp16 sign masks for coordinates 32 (2 p + s) + 16 h + r
    uint32_t om[2][8];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int pr = 0; pr < 8; ++pr) {
            const uint32_t e = 32u * (2u * p + s) + 16u * h + 2u * pr;
            om[s][pr] = (((a.dsign[e >> 5] >> (e & 31)) & 1u) << 15) |
                        (((a.dsign[(e + 1) >> 5] >> ((e + 1) & 31)) & 1u) << 31);
        }

    const int64_t stride = (int64_t)gridDim.x * VPB;
    const int64_t first = (int64_t)blockIdx.x * VPB + wave * kDecRows;
    const int64_t limit = a.n + wave * kDecRows;  // a block iteration runs while its first row < n
    stage_codes(a, first, cbuf0[wave], lane);
    // the first tile, and a tile that or whose predecessor is partial, take
    // the full wait
    bool prev_whole = false;
    for (int64_t v0 = first; v0 < limit; v0 += 2 * stride) {
        const bool w0 = v0 + kDecRows <= a.n, w1 = v0 + stride + kDecRows <= a.n;
        if (prev_whole && w0)
            dequantize_tile<true>(a, tab, A, om, cbuf0[wave], cbuf1[wave], ybuf[wave], v0, v0 + stride, lane);
        else
            dequantize_tile<false>(a, tab, A, om, cbuf0[wave], cbuf1[wave], ybuf[wave], v0, v0 + stride, lane);
        if (v0 + stride >= limit) break;
        if (w0 && w1)
            dequantize_tile<true>(a, tab, A, om, cbuf1[wave], cbuf0[wave], ybuf[wave], v0 + stride, v0 + 2 * stride,
                                  lane);
        else
            dequantize_tile<false>(a, tab, A, om, cbuf1[wave], cbuf0[wave], ybuf[wave], v0 + stride, v0 + 2 * stride,
                                   lane);
        prev_whole = w1;
    }
}

}  // namespace

hipError_t launch_quantize_kv128(const QuantArgs &a, hipStream_t s) {
    static const int per_cu = resident_blocks(k_quantize_mfma128);
    return launch(k_quantize_mfma128, dim3(grid_for(a.n, kWaves * kRowsPerWave, per_cu)), dim3(kBlock), s, a);
}

hipError_t launch_dequantize_kv128(const DequantArgs &a, hipStream_t s) {
    // two blocks per CU: the decode-shape streaming kernels ran fastest there
    static const int per_cu = resident_blocks(k_dequantize_mfma128);
    return launch(k_dequantize_mfma128, dim3(grid_for(a.n, kWaves * kDecRows, per_cu < 2 ? per_cu : 2)), dim3(kBlock),
                  s, a);
}

}  // namespace rht
