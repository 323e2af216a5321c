// rht_kernels.hip -- HIP kernels for randomized-Hadamard vector quantization
// on CDNA4 (gfx950, wave64).
//
// Method: web page "Random-rotation quantization" (brain.bigb.es): rotate each
// vector by Pi = H D / sqrt(d) (randomized Hadamard transform, "Why rotation
// works"; fast Walsh-Hadamard transform, page "TurboQuant and per-layer
// outlier-aware K", section "TurboQuant 2026"), quantize every rotated
// coordinate with one fixed N(0,1) Lloyd-Max codebook ("History", EDEN item),
// decode with Pi^T ("intro", step 3); DRIVE sign codes, the residual chain and
// rotated-domain scoring as in "History" and "Three decoders, one rotation".
//
// Register layout.  A vector of D coordinates is spread over LPV lanes of one
// wavefront, E = D / LPV coordinates per lane, held in fp32 registers for the
// whole transform.  Lane q of a vector owns the coordinates
//     e(q, r) = ((r / G) * LPV + q) * G + (r % G),   r = 0 .. E-1,
// i.e. groups of G consecutive coordinates.  G = E gives each lane one
// contiguous run (coalesced code stores); G = 8 interleaves 16-byte fp16
// chunks across the lanes of a vector (coalesced element loads).
// The Hadamard transform is a product of one butterfly stage per index bit, in
// any order: the stages on the register-index bits run in registers, the
// stages on the lane bits run across lanes.  A cross-lane stage is
//     v <- v + m * partner(v),  m = +1 on the lower lane, -1 on the upper one,
// which leaves the upper lane holding the negated value; after all lane stages
// lane q holds (-1)^popcount(q) times the true coordinate, and that factor is
// folded into the per-vector scale.
//
// Signs D: with fp16 input the sign flip, the fp16 -> fp32 conversion and the
// first butterfly stage are one v_dot2_f32_f16 per output (products by +-1
// and the sum of two fp16 values are exact in fp32).
//
// Nearest level: y16 = 16 y is mapped to a cell of a 256-entry LDS table
// (cell k covers y16 in about [k-40.5, k-39)); the entry holds the code of the
// cell's lower end and the one scaled threshold that may fall inside the cell,
// so the code is base + [y16 >= T].  The final decision compares fp32 y16 with
// the exact scaled fp32 threshold (scaling by 16 is exact).
#include "rht_device.h"

namespace rht {
namespace {

// Value of v in lane (lane ^ M); M < lanes of one vector.
template <int M>
__device__ __forceinline__ float xlane(float v) {
    const int iv = __builtin_bit_cast(int, v);
    int r;
    if constexpr (M == 1)
        r = __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true);   // quad_perm:[1,0,3,2]
    else if constexpr (M == 2)
        r = __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true);   // quad_perm:[2,3,0,1]
    else if constexpr (M == 8)
        r = __builtin_amdgcn_mov_dpp(iv, 0x128, 0xF, 0xF, true);  // row_ror:8
    else if constexpr (M == 4 || M == 16)
        r = __builtin_amdgcn_ds_swizzle(iv, (M << 10) | 0x1F);    // bit mode, xor M
    else
        r = __builtin_amdgcn_ds_bpermute((int)((lane_id() ^ M) << 2), iv);
    return __builtin_bit_cast(float, r);
}

// Sum over the LPV lanes of a vector (every lane gets the total).
template <int LPV>
__device__ __forceinline__ float vec_sum(float s) {
    if constexpr (LPV > 1) s += xlane<1>(s);
    if constexpr (LPV > 2) s += xlane<2>(s);
    if constexpr (LPV > 4) s += xlane<4>(s);
    if constexpr (LPV > 8) s += xlane<8>(s);
    if constexpr (LPV > 16) s += xlane<16>(s);
    if constexpr (LPV > 32) s += xlane<32>(s);
    return s;
}

// Butterfly stages on register-index bits FIRST.. of E registers.
template <int E, int FIRST>
__device__ __forceinline__ void fwht_regs(float (&v)[E]) {
#pragma unroll
    for (int h = 1 << FIRST; h < E; h <<= 1) {
#pragma unroll
        for (int i = 0; i < E; i += 2 * h) {
#pragma unroll
            for (int j = i; j < i + h; ++j) {
                const float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
}

// v[r] += m * v[r ^ lane M] for every register.  Partners reachable by DPP
// (xor 1, 2: quad_perm; xor 8: row_ror:8) use one v_fmac_f32_dpp per
// register.  The hardware needs two wait states between a VALU write of a
// VGPR and a DPP read of it, and the compiler cannot see into the asm, so each
// group of eight starts with s_nop 1; inside a group every instruction reads
// only its own destination, written before the group.
#define RHT_FMAC_DPP8(CTRL)                                                         \
    asm("s_nop 1\n\t"                                                               \
        "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"        \
        "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"        \
        "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"        \
        "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"        \
        "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"        \
        "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"        \
        "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"        \
        "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"              \
        : "+v"(v[r]), "+v"(v[r + 1]), "+v"(v[r + 2]), "+v"(v[r + 3]), "+v"(v[r + 4]), \
          "+v"(v[r + 5]), "+v"(v[r + 6]), "+v"(v[r + 7])                             \
        : "v"(m))

template <int M, int E>
__device__ __forceinline__ void xstage(float (&v)[E], uint32_t q) {
    const float m = (q & M) ? -1.0f : 1.0f;
    if constexpr ((M == 1 || M == 2 || M == 8) && E % 8 == 0) {
#pragma unroll
        for (int r = 0; r < E; r += 8) {
            if constexpr (M == 1)
                RHT_FMAC_DPP8("quad_perm:[1,0,3,2]");
            else if constexpr (M == 2)
                RHT_FMAC_DPP8("quad_perm:[2,3,0,1]");
            else
                RHT_FMAC_DPP8("row_ror:8");
        }
    } else {
#pragma unroll
        for (int r = 0; r < E; ++r) v[r] = fmaf(xlane<M>(v[r]), m, v[r]);
    }
}

// Butterfly stages on the lane bits; afterwards lane q holds (-1)^popcount(q)
// times the transform.
template <int LPV, int E>
__device__ __forceinline__ void fwht_lanes(float (&v)[E], uint32_t q) {
    if constexpr (LPV > 1) xstage<1>(v, q);
    if constexpr (LPV > 2) xstage<2>(v, q);
    if constexpr (LPV > 4) xstage<4>(v, q);
    if constexpr (LPV > 8) xstage<8>(v, q);
    if constexpr (LPV > 16) xstage<16>(v, q);
    if constexpr (LPV > 32) xstage<32>(v, q);
}

__device__ __forceinline__ float lane_factor(uint32_t q) {
    return (__builtin_popcount(q) & 1) ? -1.0f : 1.0f;
}

// Bit r of the result = sign bit of the coordinate held in register r.
template <int D, int G>
__device__ __forceinline__ uint64_t lane_sign_bits(const uint32_t *dsign, uint32_t q) {
    constexpr int LPV = lanes_per_vec(D), E = D / LPV, NG = E / G;
    uint64_t m = 0;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const uint32_t e0 = (gi * LPV + q) * G;
        uint64_t bits;
        if constexpr (G >= 32) {
            bits = 0;
#pragma unroll
            for (int w = 0; w < G / 32; ++w) bits |= (uint64_t)dsign[e0 / 32 + w] << (32 * w);
        } else {
            bits = (dsign[e0 >> 5] >> (e0 & 31)) & ((1u << G) - 1u);
        }
        m |= bits << (gi * G);
    }
    return m;
}

// Raw input words a lane holds for one vector: E fp16 (E/2 words) or E fp32.
template <int D, bool F16>
struct Raw {
    static constexpr int E = D / lanes_per_vec(D);
    static constexpr int W = F16 ? E / 2 : E;
};

// Load the E coordinates lane q owns of row `vec` (callers clamp the row
// index into range; results for clamped rows are never stored).
template <int D, int G, bool F16>
__device__ __forceinline__ void load_raw(const void *x, int64_t vec, uint32_t q,
                                         uint32_t (&raw)[Raw<D, F16>::W]) {
    constexpr int LPV = lanes_per_vec(D), E = D / LPV, NG = E / G;
    constexpr int EPC = F16 ? 8 : 4;  // elements per 16-byte chunk
    static_assert(G % EPC == 0, "groups are whole 16-byte chunks");
    const uint4 *row = reinterpret_cast<const uint4 *>(static_cast<const char *>(x) + vec * D * (F16 ? 2 : 4));
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
        for (int c = 0; c < G / EPC; ++c) {
            const uint4 t = row[((gi * LPV + q) * G) / EPC + c];
            const int p = (gi * G + EPC * c) / (F16 ? 2 : 1);
            raw[p] = t.x;
            raw[p + 1] = t.y;
            raw[p + 2] = t.z;
            raw[p + 3] = t.w;
        }
    }
}

// Per-lane sign words for stage0: fp16 -> packed (s_2p, s_2p+1) as +-1.0 fp16;
// fp32 -> sign-bit masks.
template <int D, bool F16>
__device__ __forceinline__ void sign_words(uint64_t lsign, uint32_t (&sw)[Raw<D, F16>::W]) {
#pragma unroll
    for (int p = 0; p < Raw<D, F16>::W; ++p) {
        if constexpr (F16)
            sw[p] = ((uint32_t)(lsign >> (2 * p)) & 1u ? 0xBC00u : 0x3C00u) |
                    (((uint32_t)(lsign >> (2 * p + 1)) & 1u ? 0xBC00u : 0x3C00u) << 16);
        else
            sw[p] = ((uint32_t)(lsign >> p) & 1u) << 31;
    }
}

// Apply D and (fp16) the first butterfly stage; return the lane's sum x_i^2.
template <int D, bool F16>
__device__ __forceinline__ float stage0(const uint32_t (&raw)[Raw<D, F16>::W],
                                        const uint32_t (&sw)[Raw<D, F16>::W],
                                        float (&v)[D / lanes_per_vec(D)]) {
    constexpr int W = Raw<D, F16>::W;
    float ss = 0.0f, ss2 = 0.0f;
#pragma unroll
    for (int p = 0; p < W; ++p) {
        if constexpr (F16) {
            v[2 * p] = dot2(raw[p], sw[p], 0.0f);
            v[2 * p + 1] = dot2(raw[p], sw[p] ^ 0x80000000u, 0.0f);
            if (p & 1)
                ss2 = dot2(raw[p], raw[p], ss2);
            else
                ss = dot2(raw[p], raw[p], ss);
        } else {
            const float f = __builtin_bit_cast(float, raw[p]);
            if (p & 1)
                ss2 = fmaf(f, f, ss2);
            else
                ss = fmaf(f, f, ss);
            v[p] = __builtin_bit_cast(float, raw[p] ^ sw[p]);
        }
    }
    return ss + ss2;
}

template <int D, int G, bool F16>
__device__ __forceinline__ float load_signed(const void *x, int64_t vec, uint32_t q, uint64_t lsign,
                                             float (&v)[D / lanes_per_vec(D)]) {
    uint32_t raw[Raw<D, F16>::W], sw[Raw<D, F16>::W];
    load_raw<D, G, F16>(x, vec, q, raw);
    sign_words<D, F16>(lsign, sw);
    return stage0<D, F16>(raw, sw, v);
}

// The same table with the two candidate levels attached, for encoders that
// also need c[code]: entry (threshold, base code, 16 c[base], 16 c[base + 1]).
template <int NCELL, int OFF>
__device__ __forceinline__ void build_lut_lev(u32x4_t *lut, const float *thr, const float *lev,
                                              int nthr) {
    for (int k = threadIdx.x; k < NCELL; k += kBlock) {
        const float lo = k == 0 ? -INFINITY : (float)(k - OFF) - 0.75f;
        const float hi = k == NCELL - 1 ? INFINITY : (float)(k - OFF) + 1.25f;
        uint32_t base = 0;
        float t_in = INFINITY;
        for (int j = 0; j < nthr; ++j) {
            const float t = 16.0f * thr[j];
            if (t < lo)
                ++base;
            else if (t < hi && t_in == INFINITY)
                t_in = t;
        }
        const uint32_t up = base < (uint32_t)nthr ? base + 1 : base;
        lut[k] = u32x4_t{__builtin_bit_cast(uint32_t, t_in), base,
                         __builtin_bit_cast(uint32_t, 16.0f * lev[base]),
                         __builtin_bit_cast(uint32_t, 16.0f * lev[up])};
    }
}

// nearest_code on the level-carrying table of NCELL cells at offset OFF; also
// returns l16 = 16 c[code].
// The table cell of y16, and the code and level within a cell: split so that
// a caller can issue several cell reads before it uses them.
template <int NCELL, int OFF, bool CLAMP>
__device__ __forceinline__ u32x4_t lut_cell(const u32x4_t *lut, float y16) {
    int b = __builtin_bit_cast(int, y16 + (8388608.0f + (float)OFF));
    if constexpr (CLAMP) b = min(max(b, 0x4B000000), 0x4B000000 + NCELL - 1);
    return lut[b - 0x4B000000];
}
// (Elements are copied to scalars before bit_cast: this compiler's bit_cast of
// an ext-vector element itself can read another element.)
__device__ __forceinline__ uint32_t code_in_cell(const u32x4_t &e, float y16, float &l16) {
    const uint32_t t = e[0], base = e[1], lo = e[2], hi = e[3];
    const bool up = y16 >= __builtin_bit_cast(float, t);
    l16 = __builtin_bit_cast(float, up ? hi : lo);
    return base + (up ? 1u : 0u);
}
template <int NCELL, int OFF, bool CLAMP>
__device__ __forceinline__ uint32_t nearest_code_lev_t(const u32x4_t *lut, float y16, float &l16) {
    return code_in_cell(lut_cell<NCELL, OFF, CLAMP>(lut, y16), y16, l16);
}
template <int D>
__device__ __forceinline__ uint32_t nearest_code_lev(const u32x4_t *lut, float y16, float &l16) {
    return nearest_code_lev_t<Lut<D>::kCells, Lut<D>::kOff, Lut<D>::kClamp>(lut, y16, l16);
}

// A level table that covers every y16 a finite d = 256 vector can produce:
// |y16| = 16 |(H D x)_i| / ||x|| <= 16 sqrt(256) = 256 (Cauchy-Schwarz; the fp32
// sums add well under one cell), so no clamp is needed.  A non-finite input
// gives an arbitrary cell index; the read then stays an LDS read (inside the
// block's allocation, or out of range, which returns zero), and no global
// access depends on it.
struct Lut256Full {
    static constexpr int kOff = 260, kCells = 520;
};

// Pack one code of width CB at group-local position t (LSB-first).
template <int CB, int WPG>
__device__ __forceinline__ void put_code(uint32_t (&w)[WPG], int t, uint32_t code) {
    const int p = t * CB, i = p / 32, sh = p % 32;
    w[i] |= code << sh;
    if (sh + CB > 32) w[i + 1] |= code >> (32 - sh);
}

template <int CB, int WPG>
__device__ __forceinline__ uint32_t get_code(const uint32_t (&w)[WPG], int t) {
    const int p = t * CB, i = p / 32, sh = p % 32;
    uint32_t c = w[i] >> sh;
    if (sh + CB > 32) c |= w[i + 1] << (32 - sh);
    return c & ((1u << CB) - 1u);
}

// Streaming accesses: the bulk inputs and outputs are touched once per launch,
// so they are read and written with the non-temporal cache policy.  With
// ordinary accesses a launch leaves dirty lines whose write-back the next
// launch pays for; measured on the bench's workloads: DRIVE encoder 0.055-0.059
// -> 0.048-0.052 ms, residual decoder 0.130 -> 0.113-0.116 ms, scoring
// 0.0171 -> 0.0155 ms.
__device__ __forceinline__ u32x4_t stream_load(const u32x4_t *p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void stream_store(T v, T *p) {
    __builtin_nontemporal_store(v, p);
}

template <int WPG>
__device__ __forceinline__ void store_words(uint32_t *dst, const uint32_t (&w)[WPG]) {
    if constexpr (WPG == 4) {
        *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if constexpr (WPG == 2) {
        *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
    } else {
#pragma unroll
        for (int i = 0; i < WPG; ++i) dst[i] = w[i];
    }
}

template <int WPG>
__device__ __forceinline__ void load_words(const uint32_t *src, uint32_t (&w)[WPG]) {
    if constexpr (WPG == 4) {
        const uint4 t = *reinterpret_cast<const uint4 *>(src);
        w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    } else if constexpr (WPG == 2) {
        const uint2 t = *reinterpret_cast<const uint2 *>(src);
        w[0] = t.x; w[1] = t.y;
    } else {
#pragma unroll
        for (int i = 0; i < WPG; ++i) w[i] = src[i];
    }
}

// ---------------------------------------------------------------------------
// LDS staging for the contiguous-run layout (G = E).  A wave's VPW rows are one
// contiguous tile of 64 * RC 16-byte chunks, RC = chunks per lane run; lane L
// owns tile chunks L*RC .. L*RC+RC-1.  Global traffic moves the tile in
// coalesced order (instruction k, lane l: chunk 64k + l); inside LDS chunk c
// of lane L's run sits at L*RC + (c ^ g(L)), g(L) = (L / (16/RC)) mod RC, so
// both the coalesced side and the per-lane run side touch 16 distinct bank
// groups per 16 lanes.
template <int D, bool F16>
struct RunStage {
    static constexpr int E = D / lanes_per_vec(D);
    static constexpr int ESZ = F16 ? 2 : 4;
    static constexpr int RC = E * ESZ / 16;  // 16-byte chunks per lane run
    static constexpr int CPR = D * ESZ / 16; // chunks per row
    static constexpr bool kOk = RC >= 2 && RC <= 16;
    static __device__ __forceinline__ uint32_t pos(uint32_t L, uint32_t c) {
        return L * RC + (c ^ ((L / (16 / RC)) % RC));
    }
};

// Coalesced global loads of the wave tile whose first row is row0 (rows past
// the end read the last row): stg[k] = tile chunk 64k + lane.
template <int D, bool F16>
__device__ __forceinline__ void tile_load(const void *x, int64_t row0, int64_t n, uint32_t lane,
                                          u32x4_t (&stg)[RunStage<D, F16>::RC]) {
    using S = RunStage<D, F16>;
#pragma unroll
    for (int k = 0; k < S::RC; ++k) {
        const uint32_t T = 64u * k + lane;
        int64_t row = row0 + T / S::CPR;
        row = row < n ? row : n - 1;
        stg[k] = stream_load(reinterpret_cast<const u32x4_t *>(static_cast<const char *>(x) + row * D * S::ESZ) + T % S::CPR);
    }
}

// Hand the coalesced chunks to their owners: stg (coalesced order) -> LDS ->
// raw (this lane's run, register order).
template <int D, bool F16>
__device__ __forceinline__ void tile_to_run(u32x4_t *buf, const u32x4_t (&stg)[RunStage<D, F16>::RC],
                                            uint32_t lane, uint32_t (&raw)[Raw<D, F16>::W]) {
    using S = RunStage<D, F16>;
#pragma unroll
    for (int k = 0; k < S::RC; ++k) {
        const uint32_t T = 64u * k + lane;
        buf[S::pos(T / S::RC, T % S::RC)] = stg[k];
    }
#pragma unroll
    for (int c = 0; c < S::RC; ++c) {
        const u32x4_t t = buf[S::pos(lane, c)];
        raw[4 * c] = t[0];
        raw[4 * c + 1] = t[1];
        raw[4 * c + 2] = t[2];
        raw[4 * c + 3] = t[3];
    }
}

// ---------------------------------------------------------------------------
// Encoder.  KIND selects the code: MSE (BITS-bit codes + ||x||), DRIVE (1-bit
// signs + S), residual chain (BITS-1 bit codes + sign plane + ||x|| + S_r).
template <int D, int G, bool F16, int BITS, int KIND>
__global__ __launch_bounds__(kBlock) void k_quantize(const QuantArgs a) {
    constexpr int LPV = lanes_per_vec(D), E = D / LPV, NG = E / G;
    constexpr int VPW = 64 / LPV, VPB = kWaves * VPW;
    constexpr bool DRIVE = (KIND == kDriveBiased || KIND == kDriveUnbiased);
    constexpr int CB = KIND == kResidual ? BITS - 1 : (DRIVE ? 1 : BITS);
    constexpr int WPG = G * CB / 32;
    static_assert(G * CB % 32 == 0, "a group's codes fill whole words");
    static_assert(KIND != kResidual || G % 32 == 0, "residual sign words need 32-coordinate groups");
    constexpr int ROWW = D * CB / 32;  // code words per row

    constexpr bool RES = KIND == kResidual, EDEN = KIND == kEden;
    __shared__ uint2 lut[DRIVE || RES || EDEN ? 1 : Lut<D>::kCells];
    __shared__ u32x4_t lutl[RES || EDEN ? Lut<D>::kCells : 1];
    if constexpr (RES || EDEN) {
        build_lut_lev<Lut<D>::kCells, Lut<D>::kOff>(lutl, a.thr, a.lev, (1 << CB) - 1);
        __syncthreads();
    } else if constexpr (!DRIVE) {
        build_lut<Lut<D>::kCells, Lut<D>::kOff>(lut, a.thr, (1 << CB) - 1);
        __syncthreads();
    }

    const uint32_t lane = lane_id(), q = lane % LPV, slot = lane / LPV, wave = threadIdx.x >> 6;
    const uint64_t lsign = lane_sign_bits<D, G>(a.dsign, q);
    const float fq = lane_factor(q);
    const float sqrt_d = __builtin_sqrtf((float)D);

    // contiguous runs (G = E) go through the LDS tile for coalesced loads;
    // not the residual encoder, whose VALU work already bounds it and which
    // loses more to the staging instructions and registers than it gains
    constexpr bool STAGE = (G == E) && RunStage<D, F16>::kOk && KIND != kResidual;
    using RS = RunStage<D, F16>;
    __shared__ u32x4_t sbuf[STAGE ? kWaves * 64 * RS::RC : 1];
    u32x4_t stg[STAGE ? RS::RC : 1];
    uint32_t sw[Raw<D, F16>::W], raw[Raw<D, F16>::W];
    sign_words<D, F16>(lsign, sw);
    const int64_t stride = (int64_t)gridDim.x * VPB;
    {
        const int64_t vec = (int64_t)blockIdx.x * VPB + wave * VPW + slot;
        if constexpr (STAGE)
            tile_load<D, F16>(a.x, (int64_t)blockIdx.x * VPB + wave * VPW, a.n, lane, stg);
        else
            load_raw<D, G, F16>(a.x, vec < a.n ? vec : a.n - 1, q, raw);
    }
    for (int64_t v0 = (int64_t)blockIdx.x * VPB; v0 < a.n; v0 += stride) {
        const int64_t vec = v0 + wave * VPW + slot;
        const bool valid = vec < a.n;
        float v[E];
        if constexpr (STAGE) tile_to_run<D, F16>(sbuf + wave * 64 * RS::RC, stg, lane, raw);
        float ss = stage0<D, F16>(raw, sw, v);
        // the next vector's loads are in flight while this one is transformed
        if constexpr (STAGE)
            tile_load<D, F16>(a.x, v0 + stride + wave * VPW, a.n, lane, stg);
        else
            load_raw<D, G, F16>(a.x, vec + stride < a.n ? vec + stride : a.n - 1, q, raw);
        fwht_regs<E, F16 ? 1 : 0>(v);
        fwht_lanes<LPV>(v, q);
        ss = vec_sum<LPV>(ss);

        if constexpr (DRIVE) {
            // bit_i = [(H D x)_i >= 0]; the register holds fq * (H D x)_i
            uint32_t w[NG][WPG];
            float l1 = 0.0f;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
                for (int i = 0; i < WPG; ++i) w[gi][i] = 0u;
#pragma unroll
                for (int t = 0; t < G; ++t) {
                    const float h = v[gi * G + t] * fq;
                    l1 += fabsf(h);
                    put_code<1, WPG>(w[gi], t, h >= 0.0f ? 1u : 0u);
                }
            }
            l1 = vec_sum<LPV>(l1);  // sum |H D x|_i = sqrt(d) ||Pi x||_1
            float S;
            if constexpr (KIND == kDriveBiased)
                S = l1 / ((float)D * sqrt_d);
            else  // ||x||^2 / ||Pi x||_1; ||x||^2 sqrt(d) could overflow where the result does not
                S = l1 > 0.0f ? ss / (l1 / sqrt_d) : 0.0f;
            if (valid) {
                uint32_t *dst = reinterpret_cast<uint32_t *>(a.codes) + vec * ROWW;
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) store_words<WPG>(dst + (gi * LPV + q) * WPG, w[gi]);
                if (q == 0) a.scale[vec] = S;
            }
        } else {
            const float nrm = sqrtf(ss);
            const float inv16 = ss > 0.0f ? fq * (16.0f / nrm) : 0.0f;
            uint32_t w[NG][WPG];
            uint32_t sw[NG][RES ? G / 32 : 1];
            float r2 = 0.0f, r1 = 0.0f, ch = 0.0f;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
                for (int i = 0; i < WPG; ++i) w[gi][i] = 0u;
                if constexpr (RES) {
                    // residual in units of y16: rho16 = y16 - 16 c[code] = 16 (h - ||x|| c) / ||x||.
                    // Sign bits enter at the bottom of a shifted word, highest t first,
                    // as 1 = negative; the word is inverted afterwards.
#pragma unroll
                    for (int i = 0; i < G / 32; ++i) {
                        uint32_t neg = 0u;
#pragma unroll
                        for (int t = 32 * i + 31; t >= 32 * i; --t) {
                            const float y16 = v[gi * G + t] * inv16;
                            float l16;
                            const uint32_t code = nearest_code_lev<D>(lutl, y16, l16);
                            put_code<CB, WPG>(w[gi], t, code);
                            const float rho = y16 - l16;
                            r2 = fmaf(rho, rho, r2);
                            r1 += fabsf(rho);
                            neg = (neg << 1) | (__builtin_bit_cast(uint32_t, rho) >> 31);
                        }
                        // a zero vector has residual 0 everywhere, whose sign bit is +1
                        sw[gi][i] = ss > 0.0f ? ~neg : 0xFFFFFFFFu;
                    }
                } else if constexpr (EDEN) {
                    // <16 c[code], y16> = 256 <c, H D x> / ||x||
#pragma unroll
                    for (int t = 0; t < G; ++t) {
                        const float y16 = v[gi * G + t] * inv16;
                        float l16;
                        put_code<CB, WPG>(w[gi], t, nearest_code_lev<D>(lutl, y16, l16));
                        ch = fmaf(l16, y16, ch);
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < G; ++t)
                        put_code<CB, WPG>(w[gi], t, nearest_code<D>(lut, v[gi * G + t] * inv16));
                }
            }
            float sr = 0.0f, se = 0.0f;
            if constexpr (EDEN) {
                // S = d ||x||^2 / <c, H D x> = d ||x|| * 256 / <16 c, y16>
                ch = vec_sum<LPV>(ch);
                se = ch > 0.0f ? (float)D * nrm * (256.0f / ch) : 0.0f;
            }
            if constexpr (RES) {
                r2 = vec_sum<LPV>(r2);
                r1 = vec_sum<LPV>(r1);
                // S_r = ||r||^2 / ||r||_1 with r = rho / sqrt(d) = (||x|| / 16) rho16 / sqrt(d)
                sr = r1 > 0.0f ? (nrm * (1.0f / 16.0f)) * (r2 / (sqrt_d * r1)) : 0.0f;
            }
            if (valid) {
                uint32_t *dst = reinterpret_cast<uint32_t *>(a.codes) + vec * ROWW;
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) store_words<WPG>(dst + (gi * LPV + q) * WPG, w[gi]);
                if constexpr (KIND == kResidual) {
                    uint32_t *sd = reinterpret_cast<uint32_t *>(a.signs) + vec * (D / 32);
#pragma unroll
                    for (int gi = 0; gi < NG; ++gi)
                        store_words<G / 32>(sd + (gi * LPV + q) * (G / 32), sw[gi]);
                    if (q == 0) a.res_scale[vec] = sr;
                }
                if (q == 0) a.scale[vec] = EDEN ? se : nrm;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Residual-chain encoder for d = 256, fp16 input, with the H_32 factor of the
// transform on MFMA.  H_256 = H_8 (x) H_32 over the split e = 32 a + b (a is
// the high index, Sylvester order).  A wave works on tiles of 16 vectors; for
// each input block a' one v_mfma_f32_16x16x32_f16 per half computes
// H_32 (D x)_{a'} with the 16 vectors as columns (K = 32 = the whole block):
// lane l (vector j = l % 16, g = l / 16) supplies the fp16 coordinates
// 32 a' + 8 g .. +8 of vector j (signs D applied by XOR), and the A rows are
// permuted so that accumulator register r of half mh holds output coordinate
// b = 8 g + 4 mh + r.  The H_8 factor is three add/sub stages across the eight
// blocks in registers; lane (j, g) ends with coordinates 32 a + 8 g .. +8 of
// vector j for every a: CB whole bytes of codes and one byte of signs per
// block, staged through LDS into coalesced row stores.
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kR256Rows = 16;  // vectors per wave tile

__device__ __forceinline__ floatx4 mfma16x16x32(u32x4_t a, u32x4_t b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
                                                  0, 0, 0);
}

// Staging of a wave tile (16 x 256 fp16 = 8 KiB) in LDS, filled by direct
// global -> LDS copies.  The 16-byte chunk c of tile row r sits at chunk
// position c ^ r of the row (r < 16), so that the 16 rows a read instruction
// touches at one chunk index land in distinct banks.  Copy instruction k fills
// 1 KiB: tile rows 2k and 2k + 1, one chunk position per lane.  The copies go
// through a buffer resource that spans the tile's rows below n, so rows past
// the end read as zeros (they are transformed but never stored).
typedef __attribute__((address_space(3))) void lds_void_r;
constexpr int kR256TileBytes = kR256Rows * 512;

__device__ __forceinline__ void stage_res256(const uint16_t *x, int64_t row0, int64_t n, char *lds_tile,
                                             uint32_t lane) {
    const int64_t rows = n - row0 < kR256Rows ? n - row0 : kR256Rows;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(x + row0 * 256), (short)0, (int)(rows * 512),
                                          kRawBufferWord3);
    // row r = 2k + h (h = lane / 32), chunk position p = lane % 32, source
    // chunk p ^ r: byte 512 r + 16 (p ^ r) = (q ^ 32k) + 1024k with
    // q = 512 h + 16 (p ^ h)
    const uint32_t h = lane >> 5, q = 512u * h + 16u * ((lane & 31u) ^ h);
#pragma unroll
    for (int k = 0; k < 8; ++k)
        // cache policy: non-temporal (each input byte is read once)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_r *)(lds_tile + 1024 * k), 16,
                                                 (q ^ (32u * k)) + 1024u * k, 0, 0, 2);
}
// The staged chunk c of row r.
__device__ __forceinline__ u32x4_t staged_chunk(const char *lds_tile, uint32_t r, uint32_t c) {
    return *reinterpret_cast<const u32x4_t *>(lds_tile + 512 * r + 16 * (c ^ (r & 15u)));
}

// Stage-1 codebooks of 1 or 2 bits have equally spaced thresholds: {0} and
// {-t, 0, t} (the codebook is symmetric).  With step = t (2 bits) or 1 (1 bit)
// and v = y / step + off, off = 1 (2 bits) or 0 (1 bit), threshold k sits at
// v = k exactly, so floor(v) alone picks the code: cell i = floor(v) holds
// code clamp(i + 1, 0, 2^CB - 1).  A value exactly at a threshold lands in the
// cell above it, as the nearest-level rule breaks ties; y = 0 gives v = off
// exactly.  The table stores (code, 16 c[code]) for cells -kEvenLow ..
// kEvenCells - kEvenLow - 1, which covers |y| <= sqrt(256) = 16 (the largest
// rotated coordinate of a normalized d = 256 vector) for any step >= 0.9.
// It is held once per position t = 0..7 of a code in its group of eight, with
// the code already shifted to bit CB t, so a group's codes combine by OR alone.
constexpr int kEvenLow = 20, kEvenCells = 44;

template <int CB>
__device__ __forceinline__ void build_even_table(uint2 (*tab)[kEvenCells], const float *lev) {
    constexpr int kMaxCode = (1 << CB) - 1;
    for (int i = threadIdx.x; i < 8 * kEvenCells; i += kBlock) {
        const int t = i / kEvenCells, k = i % kEvenCells;
        const int code = min(max(k - kEvenLow + 1, 0), kMaxCode);
        tab[t][k] = make_uint2((uint32_t)code << (CB * t), __builtin_bit_cast(uint32_t, 16.0f * lev[code]));
    }
}

// floor(v) as an integer (one v_cvt_flr_i32_f32)
__device__ __forceinline__ int floor_to_int(float v) {
    int i;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(i) : "v"(v));
    return i;
}

// At most 168 VGPRs (three waves per SIMD): the input rows come through LDS,
// so no registers hold the next tile, and the D masks are read from LDS.
// Measured on the 2^20 x 256 fp16 2+1-bit workload: 0.146 ms with the rows
// prefetched into registers (222 VGPRs, two waves per SIMD), 0.131 ms staged,
// 0.124 ms with the pre-shifted code table and bounded buffer copies.
template <int CB>
__global__ __launch_bounds__(kBlock, 3) void k_residual_quantize_mfma256(const QuantArgs a) {
    constexpr int D = 256, VPB = kWaves * kR256Rows;
    constexpr int CROW = D * CB / 8, SROW = D / 8;  // code and sign bytes per row
    using LT = Lut256Full;
    constexpr bool kEven = CB <= 2;
    // the nearest-level table: the floor-indexed one for 1- and 2-bit codes,
    // the threshold-carrying one otherwise
    __shared__ u32x4_t lutl[kEven ? 1 : LT::kCells];
    __shared__ uint2 etab[kEven ? 8 : 1][kEvenCells];
    __shared__ __attribute__((aligned(16))) char xtile[kWaves][kR256TileBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ctile[kWaves][kR256Rows * CROW];
    __shared__ __attribute__((aligned(16))) uint8_t stile[kWaves][kR256Rows * SROW];
    // D as XOR masks on the fp16 sign bits of coordinates 32 a + 8 g + t, one
    // 16-byte mask per (g, a)
    __shared__ u32x4_t smask[4][8];
    if constexpr (kEven)
        build_even_table<CB>(etab, a.lev);
    else
        build_lut_lev<LT::kCells, LT::kOff>(lutl, a.thr, a.lev, (1 << CB) - 1);
    if (threadIdx.x < 32) {
        const uint32_t gg = threadIdx.x >> 3, blk = threadIdx.x & 7u;
        const uint32_t bits8 = (a.dsign[blk] >> (8 * gg)) & 0xFFu;
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
            w[p] = (((bits8 >> (2 * p)) & 1u) << 15) | (((bits8 >> (2 * p + 1)) & 1u) << 31);
        smask[gg][blk] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
    __syncthreads();
    // v = y16 * estep + eoff (y16 = 16 y)
    const float estep = CB == 2 ? 1.0f / (16.0f * a.thr[2]) : 1.0f / 16.0f;
    const float eoff = CB == 2 ? 1.0f : 0.0f;

    const uint32_t lane = lane_id(), j = lane & 15u, g = lane >> 4;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // A operands: row rho = l % 16 of half mh is output coordinate b = 8 (rho / 4) + 4 mh + rho % 4,
    // K index k = 8 g + t
    u32x4_t A[2];
#pragma unroll
    for (int mh = 0; mh < 2; ++mh) {
        const uint32_t b = 8u * (j >> 2) + 4u * mh + (j & 3u);
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
            const uint32_t k0 = 8u * g + t, k1 = k0 + 1;
            w[t / 2] = ((__builtin_popcount(b & k0) & 1u) ? 0xBC00u : 0x3C00u) |
                       (((__builtin_popcount(b & k1) & 1u) ? 0xBC00u : 0x3C00u) << 16);
        }
        A[mh] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
    char *xt = xtile[wave];
    const float sqrt_d = 16.0f;
    const uint16_t *x = static_cast<const uint16_t *>(a.x);
    uint8_t *ct = ctile[wave];
    uint8_t *st = stile[wave];

    const int64_t stride = (int64_t)gridDim.x * VPB;
    const int64_t first = (int64_t)blockIdx.x * VPB + wave * kR256Rows;
    // one staging buffer per wave: the next tile's rows are copied in as soon
    // as this tile's rows have been read out of it, and land while this tile
    // is transformed and quantized
    if (first < a.n) stage_res256(x, first, a.n, xt, lane);
    for (int64_t v0 = first; v0 < a.n; v0 += stride) {
        // the copies into xt have landed (this also waits for the previous
        // tile's stores, which share the counter)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // ||x||^2 of vector j from the fp16 data (this lane: 64 of its coordinates)
        float ss = 0.0f, ss2 = 0.0f;
        floatx4 c[8][2];
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
            const u32x4_t raw = staged_chunk(xt, j, 4u * blk + g);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                if (p & 1)
                    ss2 = dot2(raw[p], raw[p], ss2);
                else
                    ss = dot2(raw[p], raw[p], ss);
            }
            const u32x4_t bsigned = raw ^ smask[g][blk];
            c[blk][0] = mfma16x16x32(A[0], bsigned, floatx4{0.0f, 0.0f, 0.0f, 0.0f});
            c[blk][1] = mfma16x16x32(A[1], bsigned, floatx4{0.0f, 0.0f, 0.0f, 0.0f});
        }
        // every read of xt has returned before the next tile's copies overwrite it
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (v0 + stride < a.n) stage_res256(x, v0 + stride, a.n, xt, lane);
        ss += ss2;
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        // H_8 across the blocks
#pragma unroll
        for (int hs = 1; hs < 8; hs <<= 1)
#pragma unroll
            for (int blk = 0; blk < 8; ++blk)
                if (!(blk & hs)) {
#pragma unroll
                    for (int mh = 0; mh < 2; ++mh) {
                        const floatx4 u = c[blk][mh], v = c[blk + hs][mh];
                        c[blk][mh] = u + v;
                        c[blk + hs][mh] = u - v;
                    }
                }

        const float nrm = sqrtf(ss);
        const float inv16 = ss > 0.0f ? 16.0f / nrm : 0.0f;
        const float ev = inv16 * estep;
        // a zero vector has residual 0 everywhere, whose sign bit is +1
        const uint32_t live = ss > 0.0f ? 0xFFFFFFFFu : 0u;
        float r2 = 0.0f, r1 = 0.0f;
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
            // coordinates 32 blk + 8 g + 4 mh + r, in order t = 4 mh + r
            uint32_t code = 0u, neg = 0u;
            if constexpr (kEven) {
                // the eight table reads of a block are issued together, then used
                uint2 e[8];
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    e[t] = etab[t][floor_to_int(fmaf(c[blk][t >> 2][t & 3], ev, eoff)) + kEvenLow];
                code = (e[0].x | e[1].x | e[2].x) | (e[3].x | e[4].x | e[5].x) | (e[6].x | e[7].x);
#pragma unroll
                for (int t = 7; t >= 0; --t) {
                    const float rho = fmaf(c[blk][t >> 2][t & 3], inv16, -__builtin_bit_cast(float, e[t].y));
                    r2 = fmaf(rho, rho, r2);
                    r1 += fabsf(rho);
                    neg = (neg << 1) | (__builtin_bit_cast(uint32_t, rho) >> 31);
                }
            } else {
                float y[8];
                u32x4_t e[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    y[t] = c[blk][t >> 2][t & 3] * inv16;
                    e[t] = lut_cell<LT::kCells, LT::kOff, false>(lutl, y[t]);
                }
#pragma unroll
                for (int t = 7; t >= 0; --t) {
                    const float y16 = y[t];
                    float l16;
                    const uint32_t cd = code_in_cell(e[t], y16, l16);
                    code |= cd << (CB * t);
                    const float rho = y16 - l16;
                    r2 = fmaf(rho, rho, r2);
                    r1 += fabsf(rho);
                    neg = (neg << 1) | (__builtin_bit_cast(uint32_t, rho) >> 31);
                }
            }
            // ~(neg & live) in one v_bitop3 (truth table over bit pairs:
            // 1 unless both are 1)
            const uint32_t sbits = __builtin_amdgcn_bitop3_b32(neg, live, 0u, 0x3F);
            uint8_t *cp = ct + j * CROW + CB * (4 * blk + g);
            if constexpr (CB == 2)
                *reinterpret_cast<uint16_t *>(cp) = (uint16_t)code;
            else
#pragma unroll
                for (int by = 0; by < CB; ++by) cp[by] = (uint8_t)(code >> (8 * by));
            st[j * SROW + 4 * blk + g] = (uint8_t)sbits;
        }
        r2 += __shfl_xor(r2, 16);
        r2 += __shfl_xor(r2, 32);
        r1 += __shfl_xor(r1, 16);
        r1 += __shfl_xor(r1, 32);
        const float sr = r1 > 0.0f ? (nrm * (1.0f / 16.0f)) * (r2 / (sqrt_d * r1)) : 0.0f;
        if (g == 0 && v0 + j < a.n) {
            a.scale[v0 + j] = nrm;
            a.res_scale[v0 + j] = sr;
        }
        // coalesced copy-out of the code and sign tiles (16-byte pieces)
        constexpr int CPIECES = kR256Rows * CROW / 16, SPIECES = kR256Rows * SROW / 16;
#pragma unroll
        for (int k = 0; k < (CPIECES + 63) / 64; ++k) {
            const uint32_t pc = 64u * k + lane;
            if (pc < (uint32_t)CPIECES) {
                const uint32_t r = pc / (CROW / 16);
                const u32x4_t val = reinterpret_cast<const u32x4_t *>(ct)[pc];
                if (v0 + r < a.n) stream_store(val, reinterpret_cast<u32x4_t *>(a.codes + v0 * CROW) + pc);
            }
        }
        if (lane < (uint32_t)SPIECES) {
            const uint32_t r = lane / (SROW / 16);
            const u32x4_t val = reinterpret_cast<const u32x4_t *>(st)[lane];
            if (v0 + r < a.n) stream_store(val, reinterpret_cast<u32x4_t *>(a.signs + v0 * SROW) + lane);
        }
    }
    // no staged copy is left in flight when the wave ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// Residual-chain decoder for d = 256 with fp16 output, H_32 on MFMA.
// x^ = D H z with z = (||x|| / d) c[code] + (S_r / sqrt(d)) sigma splits by
// linearity into two products per block a, with the 16 vectors of a wave tile
// as the columns of v_mfma_f32_16x16x32_f16: P = H_32 c (each level enters as
// its fp16 hi and lo parts in neighbouring K slots, so the fp32 level is
// exact) and Q = H_32 sigma (+-1, exact).  Lane (j, g) combines
// (||x_j|| / d) P + (S_r,j / sqrt(d)) Q for output coordinates 32 a + 8 g .. +8,
// runs H_8 across the blocks in registers and applies D as an XOR on the fp16
// sign bits.  Lookup tables turn a group of four codes into the {hi, hi, lo, lo}
// operand words and a sign byte into eight +-1 halves.
//
// Memory: a tile's code rows, sign rows, norms and residual scales reach LDS by
// direct global -> LDS copies, and its fp16 rows leave through an LDS tile in
// stores of two whole rows per instruction.  The copies for tile t + 1 are
// issued when tile t starts; the wave waits for them (vmcnt(0)) only after
// tile t's output is in LDS and before its global stores, so the wait covers
// the copies and the stores of tile t - 1, both issued a whole tile earlier.
typedef __attribute__((address_space(3))) void lds_void_t;

// Operand A of the decoder's products: row rho of half mh is output coordinate
// 8 (rho / 4) + 4 mh + rho % 4; K slot t of lane group g is input coordinate
// 8 g + t (sign product, h < 0) or 8 g + 4 h + (t & 3) (level product of code
// group h: hi parts in slots t < 4, lo parts in t >= 4).
__device__ __forceinline__ u32x4_t res256_operand(uint32_t j, uint32_t g, int mh, int h) {
    const uint32_t bo = 8u * (j >> 2) + 4u * mh + (j & 3u);
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
        uint32_t pair = 0u;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t tt = t + u;
            const uint32_t bi = h < 0 ? 8u * g + tt : 8u * g + 4u * h + (tt & 3u);
            pair |= ((__builtin_popcount(bo & bi) & 1u) ? 0xBC00u : 0x3C00u) << (16 * u);
        }
        w[t / 2] = pair;
    }
    return u32x4_t{w[0], w[1], w[2], w[3]};
}

// 16-byte chunk position of chunk c of tile row r in a staged tile with NC
// chunks per row (the rows of one 64-bank window land on distinct banks).
template <int NC>
__device__ __forceinline__ uint32_t rd_chunk(uint32_t r, uint32_t c) {
    return NC * r + (c ^ ((r * NC / 16u) & (NC - 1u)));
}

// Direct global -> LDS copy of the 16 rows at row0 (ROWB bytes each; rows past
// the end repeat the last row).  Lane l fills chunk position l.
template <int ROWB>
__device__ __forceinline__ void rd_stage(const uint8_t *src, int64_t row0, int64_t n, uint8_t *tile, uint32_t lane) {
    constexpr int NC = ROWB / 16;
    if (lane < 16u * NC) {
        const uint32_t r = lane / NC, cpos = lane % NC;
        const uint32_t c = cpos ^ ((r * NC / 16u) & (NC - 1u));
        const int64_t row = row0 + r < n ? row0 + r : n - 1;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4 *>(src + row * ROWB) + c,
                                         (lds_void_t *)tile, 16, 0, 0);
    }
}

// Direct copy of the norms and residual scales of the 16 rows at row0 into ft
// (lane l < 16: ||x|| of row l; 16 <= l < 32: S_r of row l - 16; rows past the
// end repeat the last row).
__device__ __forceinline__ void rd_stage_scales(const DequantArgs &a, int64_t row0, float *ft, uint32_t lane) {
    const uint32_t r = lane % kR256Rows;
    const int64_t row = row0 + r < a.n ? row0 + r : a.n - 1;
    if (lane < (uint32_t)kR256Rows)
        __builtin_amdgcn_global_load_lds(a.scale + row, (lds_void_t *)ft, 4, 0, 0);
    else if (lane < 2u * kR256Rows)
        __builtin_amdgcn_global_load_lds(a.res_scale + row, (lds_void_t *)ft, 4, 0, 0);
}

// Byte B (or the 16-bit word at B) of tile row r.
template <int ROWB>
__device__ __forceinline__ uint32_t rd_byte(const uint8_t *tile, uint32_t r, uint32_t B) {
    return tile[16u * rd_chunk<ROWB / 16>(r, B / 16u) + B % 16u];
}
template <int ROWB>
__device__ __forceinline__ uint32_t rd_u16(const uint8_t *tile, uint32_t r, uint32_t B) {
    return *reinterpret_cast<const uint16_t *>(tile + 16u * rd_chunk<ROWB / 16>(r, B / 16u) + B % 16u);
}

template <int CB>
struct Rd256Smem {
    static constexpr int kGroups = 1 << (4 * CB);            // four codes per table index
    static constexpr int kCRow = 256 * CB / 8, kSRow = 32;   // code and sign bytes per row
    u32x4_t lev[kGroups];
    u32x4_t sgn[256];
    u32x4_t om[32];                                         // [a][g]: D on coordinates 32 a + 8 g .. +8
    uint8_t c[kWaves][kR256Rows * kCRow];
    uint8_t s[kWaves][kR256Rows * kSRow];
    float f[kWaves][2 * kR256Rows];                         // ||x|| then S_r of the staged rows
    u32x4_t y[kWaves][kR256Rows * 32];                      // fp16 output tile, 16-byte chunks
};

// Waits on this wave's memory counters.  The direct global -> LDS copies are
// not reliably ordered by the compiler against LDS reads of the same buffer,
// so the kernel orders them itself: vmcnt(0) before the staged data is read,
// lgkmcnt(0) (those reads done) before the buffer is refilled.  The "memory"
// clobber keeps the compiler from moving memory accesses across either wait.
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lgkm() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// The staged inputs lane (j, g) needs: code bits and sign byte of vector j for
// coordinates 32 a + 8 g .. +8 (every block a), its norm and residual scale.
template <int CB>
__device__ __forceinline__ void rd256_fetch(const uint8_t *ct, const uint8_t *st, const float *ft, uint32_t j,
                                            uint32_t g, uint32_t (&cw)[8], uint32_t (&sw)[8], float &sc, float &rs) {
    constexpr int CROW = Rd256Smem<CB>::kCRow, SROW = Rd256Smem<CB>::kSRow;
    wait_vm();
#pragma unroll
    for (int a8 = 0; a8 < 8; ++a8) {
        cw[a8] = CB == 2 ? rd_u16<CROW>(ct, j, 8u * a8 + 2u * g) : rd_byte<CROW>(ct, j, 4u * a8 + g);
        sw[a8] = rd_byte<SROW>(st, j, 4u * a8 + g);
    }
    sc = ft[j];
    rs = ft[kR256Rows + j];
}

// One tile's arithmetic: the level and sign products per block, the per-vector
// combination and H_8 across the blocks; z[a][mh][r] is output coordinate
// 32 a + 8 g + 4 mh + r of vector j (before D).
template <int CB>
__device__ __forceinline__ void rd256_math(const Rd256Smem<CB> &sm, const u32x4_t (&Ac)[2][2], const u32x4_t (&As)[2],
                                           const uint32_t (&cw)[8], const uint32_t (&sw)[8], float sc, float rs,
                                           floatx4 (&z)[8][2]) {
    constexpr int D = 256;
    constexpr uint32_t GMASK = Rd256Smem<CB>::kGroups - 1;
    const float alpha = sc * (1.0f / D), beta = rs * (1.0f / 16.0f);  // 1 / sqrt(256)
#pragma unroll
    for (int a8 = 0; a8 < 8; ++a8) {
        const u32x4_t b0 = sm.lev[cw[a8] & GMASK];
        const u32x4_t b1 = sm.lev[(cw[a8] >> (4 * CB)) & GMASK];
        const u32x4_t bs = sm.sgn[sw[a8]];
#pragma unroll
        for (int mh = 0; mh < 2; ++mh) {
            floatx4 p = mfma16x16x32(Ac[mh][0], b0, floatx4{0.0f, 0.0f, 0.0f, 0.0f});
            p = mfma16x16x32(Ac[mh][1], b1, p);
            const floatx4 q = mfma16x16x32(As[mh], bs, floatx4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
            for (int r = 0; r < 4; ++r) z[a8][mh][r] = fmaf(alpha, p[r], beta * q[r]);
        }
    }
#pragma unroll
    for (int hs = 1; hs < 8; hs <<= 1)
#pragma unroll
        for (int a8 = 0; a8 < 8; ++a8)
            if (!(a8 & hs)) {
#pragma unroll
                for (int mh = 0; mh < 2; ++mh) {
                    const floatx4 u = z[a8][mh], v = z[a8 + hs][mh];
                    z[a8][mh] = u + v;
                    z[a8 + hs][mh] = u - v;
                }
            }
}

// fp16 with D applied, into the wave's LDS output tile (chunk c of row r at
// 32 r + (c ^ r)).
template <int CB>
__device__ __forceinline__ void rd256_to_tile(const Rd256Smem<CB> &sm, u32x4_t *yt, const floatx4 (&z)[8][2],
                                              uint32_t j, uint32_t g) {
#pragma unroll
    for (int a8 = 0; a8 < 8; ++a8) {
        const u32x4_t om = sm.om[4 * a8 + g];
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const _Float16 lo = (_Float16)z[a8][p >> 1][2 * (p & 1)];
            const _Float16 hi = (_Float16)z[a8][p >> 1][2 * (p & 1) + 1];
            o[p] = ((uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16)) ^
                   om[p];
        }
        yt[32u * j + ((4u * a8 + g) ^ j)] = u32x4_t{o[0], o[1], o[2], o[3]};
    }
}

// Copy-out of the LDS output tile: instruction k stores rows 2k and 2k + 1 whole.
__device__ __forceinline__ void rd256_flush(const DequantArgs &a, const u32x4_t *yt, int64_t v0, uint32_t lane) {
    u32x4_t *y = static_cast<u32x4_t *>(a.y);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t r = 2u * k + (lane >> 5), c = lane & 31u;
        const u32x4_t val = yt[32u * r + (c ^ r)];
        if (v0 + r < a.n) stream_store(val, y + (v0 + r) * 32 + c);
    }
}

template <int CB>
__global__ __launch_bounds__(kBlock) void k_residual_dequantize_mfma256(const DequantArgs a) {
    constexpr int VPB = kWaves * kR256Rows, CROW = Rd256Smem<CB>::kCRow, SROW = Rd256Smem<CB>::kSRow;
    constexpr int NG = Rd256Smem<CB>::kGroups;
    __shared__ __attribute__((aligned(16))) Rd256Smem<CB> sm;
    for (uint32_t k = threadIdx.x; k < (uint32_t)NG; k += kBlock) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float c = a.lev[(k >> (CB * s)) & ((1u << CB) - 1u)];
            const _Float16 h = (_Float16)c, l = (_Float16)(c - (float)h);
            hw[s] = __builtin_bit_cast(uint16_t, h);
            lw[s] = __builtin_bit_cast(uint16_t, l);
        }
        sm.lev[k] = u32x4_t{hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16), lw[0] | (lw[1] << 16), lw[2] | (lw[3] << 16)};
    }
    {
        static_assert(kBlock == 256, "one sign byte per thread");
        const uint32_t sb = threadIdx.x;
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
            w[p] = (((sb >> (2 * p)) & 1u) ? 0x3C00u : 0xBC00u) | ((((sb >> (2 * p + 1)) & 1u) ? 0x3C00u : 0xBC00u) << 16);
        sm.sgn[sb] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
    if (threadIdx.x < 32) {
        const uint32_t a8 = threadIdx.x >> 2, g = threadIdx.x & 3u;
        const uint32_t bits8 = (a.dsign[a8] >> (8 * g)) & 0xFFu;
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) w[p] = (((bits8 >> (2 * p)) & 1u) << 15) | (((bits8 >> (2 * p + 1)) & 1u) << 31);
        sm.om[threadIdx.x] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
    __syncthreads();

    const uint32_t lane = lane_id(), j = lane & 15u, g = lane >> 4;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    u32x4_t Ac[2][2], As[2];
#pragma unroll
    for (int mh = 0; mh < 2; ++mh) {
        Ac[mh][0] = res256_operand(j, g, mh, 0);
        Ac[mh][1] = res256_operand(j, g, mh, 1);
        As[mh] = res256_operand(j, g, mh, -1);
    }
    const int64_t stride = (int64_t)gridDim.x * VPB;
    const int64_t first = (int64_t)blockIdx.x * VPB + wave * kR256Rows;
    if (first >= a.n) return;
    uint8_t *ct = sm.c[wave];
    uint8_t *st = sm.s[wave];
    float *ft = sm.f[wave];
    u32x4_t *yt = sm.y[wave];
    rd_stage<CROW>(a.codes, first, a.n, ct, lane);
    rd_stage<SROW>(a.signs, first, a.n, st, lane);
    rd_stage_scales(a, first, ft, lane);
    uint32_t cw[8], sw[8];
    float sc, rs;
    rd256_fetch<CB>(ct, st, ft, j, g, cw, sw, sc, rs);
    for (int64_t v0 = first; v0 < a.n; v0 += stride) {
        const int64_t v1 = v0 + stride;
        // this tile's inputs are in registers: refill the staging buffers with the next tile's
        wait_lgkm();
        if (v1 < a.n) {
            rd_stage<CROW>(a.codes, v1, a.n, ct, lane);
            rd_stage<SROW>(a.signs, v1, a.n, st, lane);
            rd_stage_scales(a, v1, ft, lane);
        }
        floatx4 z[8][2];
        rd256_math<CB>(sm, Ac, As, cw, sw, sc, rs, z);
        rd256_to_tile<CB>(sm, yt, z, j, g);
        // the next tile's inputs, after this tile's output is in LDS (which keeps the
        // arithmetic above the wait) and before its global stores
        if (v1 < a.n) rd256_fetch<CB>(ct, st, ft, j, g, cw, sw, sc, rs);
        rd256_flush(a, yt, v0, lane);
    }
}

// Codes (and residual signs) and scales lane q needs for vector `vec`.
template <int D, int G, int BITS, int KIND>
__device__ __forceinline__ void fetch_codes(const DequantArgs &a, int64_t vec, uint32_t q,
                                            uint32_t (&w)[D / lanes_per_vec(D) / G][G * (KIND == kResidual ? BITS - 1 : ((KIND == kDriveBiased || KIND == kDriveUnbiased) ? 1 : BITS)) / 32],
                                            uint32_t (&sw)[D / lanes_per_vec(D) / G][KIND == kResidual ? G / 32 : 1],
                                            float &sc, float &rs) {
    constexpr int LPV = lanes_per_vec(D), E = D / LPV, NG = E / G;
    constexpr bool DRIVE = (KIND == kDriveBiased || KIND == kDriveUnbiased);
    constexpr int CB = KIND == kResidual ? BITS - 1 : (DRIVE ? 1 : BITS);
    constexpr int WPG = G * CB / 32;
    constexpr int ROWW = D * CB / 32;
    // rows past the end read the last row; their results are never stored
    const int64_t rv = vec < a.n ? vec : a.n - 1;
    const uint32_t *src = reinterpret_cast<const uint32_t *>(a.codes) + rv * ROWW;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) load_words<WPG>(src + (gi * LPV + q) * WPG, w[gi]);
    if constexpr (KIND == kResidual) {
        const uint32_t *ss = reinterpret_cast<const uint32_t *>(a.signs) + rv * (D / 32);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) load_words<G / 32>(ss + (gi * LPV + q) * (G / 32), sw[gi]);
        rs = a.res_scale[rv];
    }
    sc = a.scale[rv];
    (void)E;
}

// ---------------------------------------------------------------------------
// Decoder: x^ = D H z with z = c[code] (scaled by ||x|| / d afterwards), z =
// +-1 (DRIVE, scaled by S / sqrt(d)), or z = c[code] ||x|| / d + S_r sigma /
// sqrt(d) (residual chain).
template <int D, int G, bool F16OUT, int BITS, int KIND>
__global__ __launch_bounds__(kBlock) void k_dequantize(const DequantArgs a) {
    constexpr int LPV = lanes_per_vec(D), E = D / LPV, NG = E / G;
    constexpr int VPW = 64 / LPV, VPB = kWaves * VPW;
    constexpr bool DRIVE = (KIND == kDriveBiased || KIND == kDriveUnbiased);
    constexpr int CB = KIND == kResidual ? BITS - 1 : (DRIVE ? 1 : BITS);
    constexpr int WPG = G * CB / 32;
    static_assert(G * CB % 32 == 0, "a group's codes fill whole words");

    // 4-bit codes are decoded a byte (two codes) at a time from a 256-entry
    // table of level pairs; other widths use the 2^CB-entry level table.
    constexpr bool PAIRS = (CB == 4 && KIND == kMse);
    __shared__ float slev[16];
    __shared__ float2 spair[PAIRS ? 256 : 1];
    if (threadIdx.x < 16) slev[threadIdx.x] = a.lev[threadIdx.x];
    if constexpr (PAIRS) spair[threadIdx.x] = make_float2(a.lev[threadIdx.x & 15], a.lev[threadIdx.x >> 4]);
    __syncthreads();

    const uint32_t lane = lane_id(), q = lane % LPV, slot = lane / LPV, wave = threadIdx.x >> 6;
    const uint64_t lsign = lane_sign_bits<D, G>(a.dsign, q);
    const float fq = lane_factor(q);
    const float inv_sqrt_d = 1.0f / __builtin_sqrtf((float)D);
    // sign-bit masks of D for the output words (fp16 pairs or single fp32)
    constexpr int NM = F16OUT ? E / 2 : E;
    constexpr bool STAGE = (G == E) && RunStage<D, F16OUT>::kOk;
    using RS = RunStage<D, F16OUT>;
    __shared__ u32x4_t sbuf[STAGE ? kWaves * 64 * RS::RC : 1];
    uint32_t omask[NM];
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        if constexpr (F16OUT)
            omask[i] = (((uint32_t)(lsign >> (2 * i)) & 1u) << 15) | (((uint32_t)(lsign >> (2 * i + 1)) & 1u) << 31);
        else
            omask[i] = ((uint32_t)(lsign >> i) & 1u) << 31;
    }

    uint32_t w[NG][WPG];
    uint32_t sw[NG][KIND == kResidual ? G / 32 : 1];
    float sc = 0.0f, rs = 0.0f;
    const int64_t stride = (int64_t)gridDim.x * VPB;
    fetch_codes<D, G, BITS, KIND>(a, (int64_t)blockIdx.x * VPB + wave * VPW + slot, q, w, sw, sc, rs);
    for (int64_t v0 = (int64_t)blockIdx.x * VPB; v0 < a.n; v0 += stride) {
        const int64_t vec = v0 + wave * VPW + slot;
        const bool valid = vec < a.n;
        float v[E];
        float alpha;
        if constexpr (DRIVE) {
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int t = 0; t < G; ++t) v[gi * G + t] = get_code<1, WPG>(w[gi], t) ? 1.0f : -1.0f;
            alpha = fq * sc * inv_sqrt_d;
        } else if constexpr (KIND == kResidual) {
            const float a0 = sc * (1.0f / D), s0 = rs * inv_sqrt_d;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int t = 0; t < G; ++t) {
                    const float sgn = (sw[gi][t / 32] >> (t % 32)) & 1u ? s0 : -s0;
                    v[gi * G + t] = fmaf(slev[get_code<CB, WPG>(w[gi], t)], a0, sgn);
                }
            alpha = fq;
        } else if constexpr (PAIRS) {
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int i = 0; i < WPG; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float2 l2 = spair[(w[gi][i] >> (8 * j)) & 0xFFu];
                        v[gi * G + 8 * i + 2 * j] = l2.x;
                        v[gi * G + 8 * i + 2 * j + 1] = l2.y;
                    }
            alpha = fq * sc * (1.0f / D);
        } else {
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int t = 0; t < G; ++t) v[gi * G + t] = slev[get_code<CB, WPG>(w[gi], t)];
            alpha = fq * sc * (1.0f / D);
        }
        // the next vector's codes load while this one is decoded
        fetch_codes<D, G, BITS, KIND>(a, vec + stride, q, w, sw, sc, rs);
        fwht_regs<E, 0>(v);
        fwht_lanes<LPV>(v, q);
        if constexpr (STAGE) {
            // run chunks -> LDS tile -> coalesced global stores
            u32x4_t *buf = sbuf + wave * 64 * RS::RC;
#pragma unroll
            for (int c = 0; c < RS::RC; ++c) {
                uint32_t o[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if constexpr (F16OUT) {
                        const int r = 8 * c + 2 * k;
                        const _Float16 lo = (_Float16)(v[r] * alpha);
                        const _Float16 hi = (_Float16)(v[r + 1] * alpha);
                        o[k] = ((uint32_t)__builtin_bit_cast(uint16_t, lo) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16)) ^ omask[r / 2];
                    } else {
                        const int r = 4 * c + k;
                        o[k] = __builtin_bit_cast(uint32_t, v[r] * alpha) ^ omask[r];
                    }
                }
                buf[RS::pos(lane, c)] = u32x4_t{o[0], o[1], o[2], o[3]};
            }
            const int64_t row0 = v0 + wave * VPW;
            char *ybase = static_cast<char *>(a.y);
#pragma unroll
            for (int k = 0; k < RS::RC; ++k) {
                const uint32_t T = 64u * k + lane;
                const u32x4_t val = buf[RS::pos(T / RS::RC, T % RS::RC)];
                const int64_t row = row0 + T / RS::CPR;
                if (row < a.n) stream_store(val, reinterpret_cast<u32x4_t *>(ybase + row * D * RS::ESZ) + T % RS::CPR);
            }
        } else if (valid) {
            if constexpr (F16OUT) {
                uint4 *row = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.y) + vec * D);
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
                    for (int c = 0; c < G / 8; ++c) {
                        uint32_t o[4];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const int r = gi * G + 8 * c + 2 * k;
                            const _Float16 lo = (_Float16)(v[r] * alpha);
                            const _Float16 hi = (_Float16)(v[r + 1] * alpha);
                            const uint32_t pk = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                                                ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                            o[k] = pk ^ omask[r / 2];
                        }
                        row[((gi * LPV + q) * G) / 8 + c] = make_uint4(o[0], o[1], o[2], o[3]);
                    }
                }
            } else {
                uint4 *row = reinterpret_cast<uint4 *>(static_cast<float *>(a.y) + vec * D);
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
                    for (int c = 0; c < G / 4; ++c) {
                        uint32_t o[4];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const int r = gi * G + 4 * c + k;
                            o[k] = __builtin_bit_cast(uint32_t, v[r] * alpha) ^ omask[r];
                        }
                        row[((gi * LPV + q) * G) / 4 + c] = make_uint4(o[0], o[1], o[2], o[3]);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Scoring on the codes in the rotated domain: logits = Qt * C^T scaled per key,
// Qt = (H D Q^T)^T formed once per block into LDS, C[k][i] = c[code_{k,i}]
// (MSE codes: Lloyd-Max levels, factor ||k|| / d; sign codes: +-1, factor
// S / sqrt(d)).  RES: the residual chain, C[k][i] = (||k|| / d) c[code_{k,i}]
// + (S_r / sqrt(d)) sigma_{k,i}, no further factor.
// The contraction runs on v_mfma_f32_32x32x2_f32: per wave a 64-query x
// 32-key tile (two 32x32 accumulators sharing the key operand).
// The block's queries rotated into LDS, transposed: qt[i * QS + j] = (H D q_j)_i
// (Sylvester H, unnormalized) for j < 64; rows j >= m repeat the last query.
// With qmax, qmax[j] = max_i |qt[i][j]|.
// after_load() runs once the first round's query loads are issued (a caller
// can queue its own copies behind them).
struct NoHook {
    __device__ void operator()() const {}
};

// Queries q0 .. q0 + NQ - 1 go to columns 0 .. NQ - 1 of qt.
template <int D, int QS, int NQ = 64, typename Hook = NoHook>
__device__ __forceinline__ void rotate_queries(const ScoreArgs &a, float *qt, float *qmax, int q0 = 0,
                                               Hook after_load = Hook{}) {
    constexpr int LPV = lanes_per_vec(D), E = D / LPV, VPW = 64 / LPV, VPB = kWaves * VPW;
    const uint32_t lane = lane_id(), q = lane % LPV, slot = lane / LPV, wave = threadIdx.x >> 6;
    const uint64_t lsign = lane_sign_bits<D, E>(a.dsign, q);
    const float fq = lane_factor(q);
    for (int j0 = 0; j0 < NQ; j0 += VPB) {
        const int j = j0 + wave * VPW + slot;  // column; query q0 + j
        const bool valid = q0 + j < a.m;
        float v[E];
        {
            uint32_t raw[Raw<D, false>::W], sw[Raw<D, false>::W];
            load_raw<D, E, false>(a.q, valid ? q0 + j : a.m - 1, q, raw);
            if (j0 == 0) after_load();
            sign_words<D, false>(lsign, sw);
            stage0<D, false>(raw, sw, v);
        }
        fwht_regs<E, 0>(v);
        fwht_lanes<LPV>(v, q);
        float mx = 0.0f;
#pragma unroll
        for (int r = 0; r < E; ++r) {
            v[r] *= fq;
            mx = fmaxf(mx, fabsf(v[r]));
        }
        if (j < NQ) {
#pragma unroll
            for (int r = 0; r < E; ++r) qt[(q * E + r) * QS + j] = v[r];
        }
        if (qmax) {
#pragma unroll
            for (int o = 1; o < LPV; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            if (q == 0 && j < NQ) qmax[j] = mx;
        }
    }
}

template <int D, int BITS, bool RES>
__global__ __launch_bounds__(kBlock) void k_score(const ScoreArgs a) {
    constexpr int QS = 96;  // LDS row stride of the transposed queries (bank spread)
    constexpr int ROWW = D * BITS / 32;
    __shared__ float qt[D * QS];
    __shared__ float slev[16];

    const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
    if (threadIdx.x < 16) slev[threadIdx.x] = a.lev[threadIdx.x];
    rotate_queries<D, QS>(a, qt, nullptr);
    __syncthreads();

    const uint32_t col = lane & 31u, par = lane >> 5;
    const int64_t ntiles = (a.n + 31) / 32;
    for (int64_t tile = (int64_t)blockIdx.x * kWaves + wave; tile < ntiles;
         tile += (int64_t)gridDim.x * kWaves) {
        const int64_t key = tile * 32 + col;
        const bool valid = key < a.n;
        const int64_t row = valid ? key : a.n - 1;
        uint32_t w[ROWW];
        load_words<ROWW>(reinterpret_cast<const uint32_t *>(a.codes) + row * ROWW, w);
        // residual chain: B element (||x|| / d) c[code] + (S_r / sqrt(d)) sigma, so the
        // accumulator is the logit itself
        uint32_t sw[RES ? D / 32 : 1];
        float na = 0.0f, nb = 0.0f;
        if constexpr (RES) {
            load_words<D / 32>(reinterpret_cast<const uint32_t *>(a.signs) + row * (D / 32), sw);
            na = a.norms[row] * (1.0f / D);
            nb = a.res_scale[row] * (1.0f / __builtin_sqrtf((float)D));
        }
        floatx16 acc0 = {}, acc1 = {};
#pragma unroll
        for (int s = 0; s < D / 2; ++s) {
            const uint32_t c0 = get_code<BITS, ROWW>(w, 2 * s), c1 = get_code<BITS, ROWW>(w, 2 * s + 1);
            const int i = 2 * s + par;
            float b = slev[par ? c1 : c0];
            if constexpr (RES) {
                const float sg = ((sw[i >> 5] >> (i & 31)) & 1u) ? nb : -nb;
                b = fmaf(na, b, sg);
            }
            const float a0 = qt[i * QS + col], a1 = qt[i * QS + 32 + col];
            acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b, acc1, 0, 0, 0);
        }
        if (valid) {
            const float sc = RES ? 1.0f : a.norms[key] * a.key_mult;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qrow = 8 * (r / 4) + 4 * par + (r % 4);
                if (qrow < a.m) a.logits[(int64_t)qrow * a.n + key] = acc0[r] * sc;
                if (qrow + 32 < a.m) a.logits[(int64_t)(qrow + 32) * a.n + key] = acc1[r] * sc;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Scoring for d >= 512.  The rotated queries of a whole block do not fit in
// LDS at these d, so a block serves a group of QG queries (QG * d fp32 in LDS,
// QG = 32, 16, 8, 4 at d = 512 ... 4096) and the m queries take ceil(m / QG)
// groups.  A wave's lane (key col, K half par) walks its key's code row in
// chunks of 256 coordinates (whole words for every code width), so only one
// chunk of codes is in registers at a time; the contraction is
// v_mfma_f32_32x32x2_f32 as in k_score (query rows past QG repeat the group's
// last query and are not stored).  Blocks are placed so that the G groups
// scoring the same key tiles sit on one XCD (blocks are dispatched to the eight
// XCDs in turn: block b runs on XCD b % 8): the G reads of a code row after
// the first can hit that XCD's L2.
template <int N>
__device__ __forceinline__ void load_words_x4(const uint32_t *src, uint32_t (&w)[N]) {
    static_assert(N % 4 == 0, "whole 16-byte pieces");
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
        const uint4 t = reinterpret_cast<const uint4 *>(src)[k];
        w[4 * k] = t.x; w[4 * k + 1] = t.y; w[4 * k + 2] = t.z; w[4 * k + 3] = t.w;
    }
}

template <int D>
constexpr int wide_score_group() { return D >= 4096 ? 4 : 16384 / D; }

template <int D, int BITS, bool RES>
__global__ __launch_bounds__(kBlock) void k_score_wide(const ScoreArgs a) {
    constexpr int QG = wide_score_group<D>();
    constexpr int QS = QG + 1;               // LDS stride of a coordinate row of qt
    constexpr int KC = 256;                  // coordinates per chunk of a code row
    constexpr int CW = KC * BITS / 32;       // code words per chunk
    constexpr int ROWW = D * BITS / 32;      // code words per key
    static_assert(D >= 512 && CW % 4 == 0, "chunks are whole 16-byte pieces");
    __shared__ float qt[D * QS];
    __shared__ float slev[16];

    const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
    const int G = (a.m + QG - 1) / QG;
    const uint32_t b = blockIdx.x, slot = b / 8, xcd = b % 8;
    const int grp = (int)(slot % (uint32_t)G);
    const int64_t tb = (int64_t)(slot / (uint32_t)G) * 8 + xcd, ntb = gridDim.x / G;
    if (threadIdx.x < 16) slev[threadIdx.x] = a.lev[threadIdx.x];
    rotate_queries<D, QS, QG>(a, qt, nullptr, grp * QG);
    __syncthreads();

    const uint32_t col = lane & 31u, par = lane >> 5;
    const uint32_t qcol = col < (uint32_t)QG ? col : (uint32_t)QG - 1;
    const int64_t ntiles = (a.n + 31) / 32;
    for (int64_t tile = tb * kWaves + wave; tile < ntiles; tile += ntb * kWaves) {
        const int64_t key = tile * 32 + col;
        const bool valid = key < a.n;
        const int64_t row = valid ? key : a.n - 1;
        float na = 0.0f, nb = 0.0f;
        if constexpr (RES) {
            na = a.norms[row] * (1.0f / D);
            nb = a.res_scale[row] * (1.0f / __builtin_sqrtf((float)D));
        }
        const uint32_t *crow = reinterpret_cast<const uint32_t *>(a.codes) + row * ROWW;
        floatx16 acc = {};
        for (int c = 0; c < D / KC; ++c) {
            uint32_t w[CW];
            load_words_x4<CW>(crow + c * CW, w);
            uint32_t sw[RES ? KC / 32 : 4];
            if constexpr (RES)
                load_words_x4<KC / 32>(reinterpret_cast<const uint32_t *>(a.signs) + row * (D / 32) + c * (KC / 32),
                                       sw);
            const float *qc = qt + (size_t)c * KC * QS;
#pragma unroll
            for (int s = 0; s < KC / 2; ++s) {
                const uint32_t c0 = get_code<BITS, CW>(w, 2 * s), c1 = get_code<BITS, CW>(w, 2 * s + 1);
                const int i = 2 * s + (int)par;  // coordinate within the chunk
                float bv = slev[par ? c1 : c0];
                if constexpr (RES) {
                    const float sg = ((sw[i >> 5] >> (i & 31)) & 1u) ? nb : -nb;
                    bv = fmaf(na, bv, sg);
                }
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qc[i * QS + qcol], bv, acc, 0, 0, 0);
            }
        }
        if (valid) {
            const float sc = RES ? 1.0f : a.norms[key] * a.key_mult;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qrow = 8 * (r / 4) + 4 * (int)par + (r % 4);
                const int qq = grp * QG + qrow;
                if (qrow < QG && qq < a.m) stream_store(acc[r] * sc, a.logits + (int64_t)qq * a.n + key);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Scoring on the fp16 matrix cores at fp32-level accuracy (d <= 128).
// logits[q][k] = f_k 2^-e_q sum_i Qs[q][i] C[k][i]: Qs = 2^e_q (H D q) with e_q
// putting the largest |coordinate| of query q in [2^14, 2^15), split into fp16
// hi and lo parts Qh + Ql; C[k][i] = c[code_{k,i}] split the same way (exact
// for +-1 levels).  Each 32 x 32 x 16 step accumulates Qh Ch + Qh Cl + Ql Ch on
// v_mfma_f32_32x32x16_f16 (the dropped Ql Cl is ~2^-22 of a product; EXACT
// levels skip Qh Cl).  Residual chain: a second accumulator takes
// (Qh + Ql) sigma, and f_k = ||k|| / d on the levels, S_r / sqrt(d) on the
// signs.  A wave owns the 32 queries of one half (its A operands stay in
// registers) and walks 32-key tiles; K slot t of lane half h in step s is
// coordinate (d/2) h + 8 s + t, so a lane's codes are one contiguous half row.
// A pair of codes maps to its levels' fp16 hi and lo parts through an LDS table.
template <int N>
__device__ __forceinline__ void load_half_row(const uint8_t *p, uint32_t (&w)[N]) {
    // p is aligned to the largest power of two dividing both the row and half-row sizes
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int k = 0; k < N / 4; ++k) {
            const uint4 t = reinterpret_cast<const uint4 *>(p)[k];
            w[4 * k] = t.x; w[4 * k + 1] = t.y; w[4 * k + 2] = t.z; w[4 * k + 3] = t.w;
        }
    } else if constexpr (N % 2 == 0) {
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
            const uint2 t = reinterpret_cast<const uint2 *>(p)[k];
            w[2 * k] = t.x; w[2 * k + 1] = t.y;
        }
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) w[k] = reinterpret_cast<const uint32_t *>(p)[k];
    }
}

__device__ __forceinline__ floatx16 mfma32x32x16(u32x4_t a, u32x4_t b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
                                                  0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_half2(_Float16 lo, _Float16 hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// Lane step s of the key operands: B_h / B_l carry the fp16 hi / lo parts of the
// levels of coordinates (d/2) h + 8 s .. +8, from four code-pair lookups.
template <int BITS, int HW>
__device__ __forceinline__ void key_operands(const uint2 *ptab, const uint32_t (&w)[HW], int s, u32x4_t &bh,
                                             u32x4_t &bl) {
    uint2 e[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) e[p] = ptab[get_code<2 * BITS, HW>(w, 4 * s + p)];
    bh = u32x4_t{e[0].x, e[1].x, e[2].x, e[3].x};
    bl = u32x4_t{e[0].y, e[1].y, e[2].y, e[3].y};
}

// Direct global -> LDS copies of the kScoreTK key tiles from `tile` on (32 keys
// each): code rows (chunk c of row r at position NC r + (c ^ ((r / 4) % NC))
// when NC, the chunks per row, is a power of two), norms (and for the residual
// chain S_r and the sign rows).  Keys past the end repeat the last chunk / key.
constexpr int kScoreTK = 2;  // key tiles per wave item

template <int ROWB, bool RES>
__device__ __forceinline__ void stage_keys(const ScoreArgs &a, int64_t tile, uint8_t *kc, uint8_t *ks, float *kn,
                                           uint32_t lane) {
    constexpr int NC = ROWB / 16, CH = 32 * kScoreTK * NC;  // chunks per row, per item
    constexpr bool SWZ = (NC & (NC - 1)) == 0;
    const int64_t last = (a.n * ROWB) / 16 - 1;              // last code chunk of the array
#pragma unroll
    for (int k = 0; k < (CH + 63) / 64; ++k) {
        const uint32_t p = 64u * k + lane;
        if (p < (uint32_t)CH) {
            const uint32_t r = p / NC, cp = p % NC;
            const uint32_t c = SWZ ? (cp ^ ((r >> 2) & (NC - 1))) : cp;
            int64_t g = tile * (32 * NC) + r * NC + c;
            g = g < last ? g : last;
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4 *>(a.codes) + g,
                                             (lds_void_t *)(kc + 1024 * k), 16, 0, 0);
        }
    }
    static_assert(kScoreTK == 2, "one lane per key of the item");
    const int64_t key = tile * 32 + lane < a.n ? tile * 32 + lane : a.n - 1;
    __builtin_amdgcn_global_load_lds(a.norms + key, (lds_void_t *)kn, 4, 0, 0);
    if constexpr (RES) {
        __builtin_amdgcn_global_load_lds(a.res_scale + key, (lds_void_t *)(kn + 64), 4, 0, 0);
        // sign rows: 16 bytes per key (d = 128)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4 *>(a.signs) + key, (lds_void_t *)ks, 16, 0, 0);
    }
}

// Lane (key r of the item, half h)'s staged data: its half row of codes, sign
// bytes, norm and residual scale.
template <int ROWB, bool RES, int HW>
__device__ __forceinline__ void fetch_keys(const uint8_t *kc, const uint8_t *ks, const float *kn, uint32_t r,
                                           uint32_t h, uint32_t (&w)[HW], uint32_t (&sg)[2], float &fa, float &fb) {
    constexpr int NC = ROWB / 16;
    constexpr bool SWZ = (NC & (NC - 1)) == 0;
#pragma unroll
    for (int k = 0; k < HW; ++k) {
        const uint32_t byte = h * (HW * 4) + 4 * k, c = byte / 16;
        const uint32_t pos = NC * r + (SWZ ? (c ^ ((r >> 2) & (NC - 1))) : c);
        w[k] = *reinterpret_cast<const uint32_t *>(kc + 16 * pos + byte % 16);
    }
    if constexpr (RES) {
        const uint2 t = *reinterpret_cast<const uint2 *>(ks + 16 * r + 8 * h);
        sg[0] = t.x;
        sg[1] = t.y;
        fb = kn[64 + r];
    }
    fa = kn[r];
}

template <int D, int BITS, bool RES, bool EXACT>
__device__ __forceinline__ void score_tile(const uint2 *ptab, const u32x4_t *stab, const u32x4_t (&Ah)[D / 16],
                                           const u32x4_t (&Al)[D / 16], const uint32_t (&w)[D * BITS / 64],
                                           const uint32_t (&sg)[2], floatx16 &acc, floatx16 &accs) {
    constexpr int S = D / 16, HW = D * BITS / 64;
    acc = floatx16{};
    accs = floatx16{};
#pragma unroll
    for (int s = 0; s < S; ++s) {
        u32x4_t bh, bl;
        key_operands<BITS, HW>(ptab, w, s, bh, bl);
        acc = mfma32x32x16(Ah[s], bh, acc);
        if constexpr (!EXACT) acc = mfma32x32x16(Ah[s], bl, acc);
        acc = mfma32x32x16(Al[s], bh, acc);
        if constexpr (RES) {
            const u32x4_t bs = stab[(sg[s / 4] >> (8 * (s % 4))) & 0xFFu];
            accs = mfma32x32x16(Ah[s], bs, accs);
            accs = mfma32x32x16(Al[s], bs, accs);
        }
    }
}

// The 32 queries q0 .. q0 + 31 of a block rotated (H D q), each scaled by
// 2^e_q so that its largest |coordinate| lies in [2^14, 2^15), and split into
// fp16 hi and lo parts: row q of `ah` / `al` (kQRow halves apart) holds them
// for coordinates 0 .. 127; qinv[q] = 2^-e_q.  Eight lanes per query, 16
// consecutive coordinates each (the transform's bits 0-3 in registers, bits
// 4-6 across the lanes), and each lane scales and splits its own coordinates,
// so the operands need no further pass; queries past m repeat the last one.
// With eight lanes per query the four waves of a block rotate exactly its 32
// queries and each lane's butterfly chain is half as long as with four (131072
// keys: 14.6-15.4 -> 13.7-14.1 us, same logits).  after_load() runs once the
// query rows are in registers.
constexpr int kQRow = 136;  // 272-byte rows: successive rows start four banks apart

template <typename Hook>
__device__ __forceinline__ void rotate_split_queries(const ScoreArgs &a, uint16_t *ah, uint16_t *al, float *qinv,
                                                     int q0, Hook after_load) {
    // eight lanes per query, 16 consecutive coordinates each: the four waves
    // of a block rotate its 32 queries, eight each
    constexpr int D = 128, LPV = 8, E = D / LPV;
    const uint32_t lane = lane_id(), q = lane % LPV, slot = lane / LPV, wave = threadIdx.x >> 6;
    const int j = (int)(wave * (64 / LPV) + slot);  // query q0 + j
    const uint32_t lsign = (a.dsign[(E * q) >> 5] >> ((E * q) & 31)) & 0xFFFFu;
    const float fq = lane_factor(q);
    float v[E];
    {
        const int64_t row = q0 + j < a.m ? q0 + j : a.m - 1;
        const uint4 *src = reinterpret_cast<const uint4 *>(a.q + row * D) + (E / 4) * q;
#pragma unroll
        for (int c = 0; c < E / 4; ++c) {
            const uint4 t = src[c];
            const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int k = 0; k < 4; ++k)
                v[4 * c + k] = __builtin_bit_cast(float, w[k] ^ (((lsign >> (4 * c + k)) & 1u) << 31));
        }
    }
    // what after_load() issues stays behind every use of the query loads, so their
    // waits do not also cover it
    static_assert(E % 8 == 0, "eight values per ordering statement");
#pragma unroll
    for (int k = 0; k < E; k += 8)
        asm volatile("" ::"v"(v[k]), "v"(v[k + 1]), "v"(v[k + 2]), "v"(v[k + 3]), "v"(v[k + 4]), "v"(v[k + 5]),
                     "v"(v[k + 6]), "v"(v[k + 7])
                     : "memory");
    after_load();
    fwht_regs<E, 0>(v);
    fwht_lanes<LPV>(v, q);
    float mx = 0.0f;
#pragma unroll
    for (int r = 0; r < E; ++r) {
        v[r] *= fq;
        mx = fmaxf(mx, fabsf(v[r]));
    }
#pragma unroll
    for (int o = 1; o < LPV; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    int ex;
    (void)frexpf(mx, &ex);
    const int e = mx > 0.0f ? min(max(15 - ex, -126), 126) : 0;
    if (q == 0) qinv[j] = ldexpf(1.0f, -e);
    uint32_t hw[E / 2], lw[E / 2];
#pragma unroll
    for (int r = 0; r < E; r += 2) {
        const float v0 = ldexpf(v[r], e), v1 = ldexpf(v[r + 1], e);
        const _Float16 a0 = (_Float16)v0, a1 = (_Float16)v1;
        hw[r / 2] = pack_half2(a0, a1);
        lw[r / 2] = pack_half2((_Float16)(v0 - (float)a0), (_Float16)(v1 - (float)a1));
    }
    uint4 *hrow = reinterpret_cast<uint4 *>(ah + j * kQRow + E * q);
    uint4 *lrow = reinterpret_cast<uint4 *>(al + j * kQRow + E * q);
#pragma unroll
    for (int k = 0; k < E / 8; ++k) {
        hrow[k] = make_uint4(hw[4 * k], hw[4 * k + 1], hw[4 * k + 2], hw[4 * k + 3]);
        lrow[k] = make_uint4(lw[4 * k], lw[4 * k + 1], lw[4 * k + 2], lw[4 * k + 3]);
    }
}

template <int D, int BITS, bool RES, bool EXACT>
__global__ __launch_bounds__(kBlock) void k_score_mfma(const ScoreArgs a) {
    static_assert(D == 128, "a query half's operands stay in registers; code rows are whole 16-byte chunks");
    constexpr int S = D / 16;                 // K steps of 16 coordinates
    constexpr int HC = D / 2;                 // coordinates per lane half
    constexpr int HW = HC * BITS / 32;        // code words per half row
    constexpr int ROWB = D * BITS / 8;        // code bytes per key
    constexpr int KI = 32 * kScoreTK;         // keys per wave item
    // this block's 32 queries as the fp16 hi and lo parts of the A operands
    __shared__ __attribute__((aligned(16))) uint16_t qah[32 * kQRow];
    __shared__ __attribute__((aligned(16))) uint16_t qal[32 * kQRow];
    __shared__ __attribute__((aligned(16))) float qinv[32];  // 2^-e_q
    __shared__ uint2 ptab[1 << (2 * BITS)];   // code pair -> {hi parts, lo parts} of its two levels
    __shared__ u32x4_t stab[RES ? 256 : 1];   // sign byte -> eight +-1 halves
    __shared__ __attribute__((aligned(16))) uint8_t kcb[kWaves][KI * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t ksb[kWaves][RES ? KI * (D / 8) : 16];
    __shared__ float knb[kWaves][2 * KI];

    const uint32_t lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t i = lane & 31u, h = lane >> 5;
    // a block serves one half of the queries (32 each).  With two halves, blocks
    // b and b + 8 (the launch makes the grid a multiple of 16) take the same
    // items, one half each: blocks are dispatched to the eight XCDs in turn, so
    // the pair shares an XCD and the second block's code reads can hit that
    // XCD's L2.  Item group ib = 8 (b / 16) + b % 8 takes items ib, ib + grid / 2, ...
    const int RH = a.m > 32 ? 2 : 1;
    const uint32_t b = blockIdx.x;
    const int rh = RH == 2 ? (int)((b >> 3) & 1u) : 0;
    const uint32_t ib = RH == 2 ? ((b >> 4) << 3) + (b & 7u) : b;
    const int64_t gw = (int64_t)ib * kWaves + wave, nw = (int64_t)(gridDim.x / RH) * kWaves;
    const int64_t ntiles = (a.n + 31) / 32, istride = nw * kScoreTK;
    int64_t tile = gw * kScoreTK;  // first tile of this wave's item
    uint8_t *kc = kcb[wave];
    uint8_t *ks = ksb[wave];
    float *kn = knb[wave];
    for (uint32_t k = threadIdx.x; k < (1u << (2 * BITS)); k += kBlock) {
        // the levels are selected from scalar registers (a per-lane index into the
        // kernel arguments would be a vector load, and its wait would hold up the copies)
        float c0 = 0.0f, c1 = 0.0f;
#pragma unroll
        for (uint32_t t = 0; t < (1u << BITS); ++t) {
            c0 = (k & ((1u << BITS) - 1u)) == t ? a.lev[t] : c0;
            c1 = (k >> BITS) == t ? a.lev[t] : c1;
        }
        const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
        ptab[k] = make_uint2(pack_half2(h0, h1), pack_half2((_Float16)(c0 - (float)h0), (_Float16)(c1 - (float)h1)));
    }
    if constexpr (RES) {
        static_assert(kBlock == 256, "one sign byte per thread");
        const uint32_t sb = threadIdx.x;
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
            w[p] = (((sb >> (2 * p)) & 1u) ? 0x3C00u : 0xBC00u) | ((((sb >> (2 * p + 1)) & 1u) ? 0x3C00u : 0xBC00u) << 16);
        stab[sb] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
    // the first item's keys are copied while the queries are rotated
    rotate_split_queries(a, qah, qal, qinv, 32 * rh, [&] {
        if (tile < ntiles) stage_keys<ROWB, RES>(a, tile, kc, ks, kn, lane);
    });
    __syncthreads();  // every wave of the block reaches this barrier

    // A operands of this block's query half: row i is query 32 rh + i; K slot t
    // of lane half h in step s is coordinate HC h + 8 s + t
    u32x4_t Ah[S], Al[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        Ah[s] = *reinterpret_cast<const u32x4_t *>(qah + i * kQRow + HC * h + 8 * s);
        Al[s] = *reinterpret_cast<const u32x4_t *>(qal + i * kQRow + HC * h + 8 * s);
    }
    if (tile >= ntiles) return;

    uint32_t w0[HW], w1[HW], sg0[2] = {0u, 0u}, sg1[2] = {0u, 0u};
    float fa0, fa1, fb0 = 0.0f, fb1 = 0.0f;
    wait_vm();
    fetch_keys<ROWB, RES, HW>(kc, ks, kn, i, h, w0, sg0, fa0, fb0);
    fetch_keys<ROWB, RES, HW>(kc, ks, kn, 32 + i, h, w1, sg1, fa1, fb1);
    for (;;) {
        const int64_t next = tile + istride;
        wait_lgkm();  // this item's staged data is in registers
        if (next < ntiles) stage_keys<ROWB, RES>(a, next, kc, ks, kn, lane);
        floatx16 acc0, accs0, acc1, accs1;
        score_tile<D, BITS, RES, EXACT>(ptab, stab, Ah, Al, w0, sg0, acc0, accs0);
        score_tile<D, BITS, RES, EXACT>(ptab, stab, Ah, Al, w1, sg1, acc1, accs1);
        // per-key factors: ||k|| key_mult (MSE, sign), ||k|| / d and S_r / sqrt(d) (residual chain)
        const float km = RES ? 1.0f / D : a.key_mult, kr = 1.0f / __builtin_sqrtf((float)D);
        const float fa0_t = fa0 * km, fa1_t = fa1 * km, fb0_t = fb0 * kr, fb1_t = fb1 * kr;
        if (next < ntiles) {
            // the next item's data, once this item's products are issued (the wait takes
            // the accumulators as inputs) and before its stores (so it never waits on them)
            asm volatile("s_waitcnt vmcnt(0)" ::"v"(acc0[15]), "v"(acc1[15]), "v"(accs0[15]), "v"(accs1[15])
                         : "memory");
            fetch_keys<ROWB, RES, HW>(kc, ks, kn, i, h, w0, sg0, fa0, fb0);
            fetch_keys<ROWB, RES, HW>(kc, ks, kn, 32 + i, h, w1, sg1, fa1, fb1);
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            // queries 32 rh + 8 r4 + 4 h .. +4: accumulator registers 4 r4 .. +4
            const int Q0 = 32 * rh + 8 * r4 + 4 * (int)h;
            const float4 qi = *reinterpret_cast<const float4 *>(qinv + (Q0 - 32 * rh));
            const float qv[4] = {qi.x, qi.y, qi.z, qi.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = 4 * r4 + u, Q = Q0 + u;
                if (Q < a.m) {
                    const int64_t key0 = tile * 32 + i, key1 = key0 + 32;
                    float v0 = acc0[r] * fa0_t, v1 = acc1[r] * fa1_t;
                    if constexpr (RES) {
                        v0 = fmaf(accs0[r], fb0_t, v0);
                        v1 = fmaf(accs1[r], fb1_t, v1);
                    }
                    if (key0 < a.n) stream_store(v0 * qv[u], a.logits + (int64_t)Q * a.n + key0);
                    if (key1 < a.n) stream_store(v1 * qv[u], a.logits + (int64_t)Q * a.n + key1);
                }
            }
        }
        tile = next;
        if (tile >= ntiles) break;
    }
}

template <int D>
constexpr int vecs_per_block() { return kWaves * (64 / lanes_per_vec(D)); }

template <int D, int G, bool F16, int BITS, int KIND>
hipError_t run_q(const QuantArgs &a, hipStream_t s) {
    static const int per_cu = resident_blocks(k_quantize<D, G, F16, BITS, KIND>);
    return launch(k_quantize<D, G, F16, BITS, KIND>, dim3(grid_for(a.n, vecs_per_block<D>(), per_cu)),
                  dim3(kBlock), s, a);
}

// grid_for with a kernel's own cap on resident blocks per CU, below the default.
inline int capped_grid(int64_t n, int vpb, int per_cu, int cap) { return grid_for(n, vpb, min(per_cu, cap)); }

template <int D, int G, bool F16, int BITS, int KIND>
hipError_t run_dq(const DequantArgs &a, hipStream_t s) {
    static const int per_cu = resident_blocks(k_dequantize<D, G, F16, BITS, KIND>);
    // the decoder's traffic is mostly writes, and HBM write throughput drops
    // with many concurrent writers: two blocks per CU (DRIVE d = 1024 fp32
    // decode: 0.054 -> 0.052 ms)
    return launch(k_dequantize<D, G, F16, BITS, KIND>, dim3(capped_grid(a.n, vecs_per_block<D>(), per_cu, 2)),
                  dim3(kBlock), s, a);
}

template <int CB>
hipError_t run_res256_cb(const QuantArgs &a, hipStream_t s) {
    static const int per_cu = resident_blocks(k_residual_quantize_mfma256<CB>);
    return launch(k_residual_quantize_mfma256<CB>, dim3(grid_for(a.n, kWaves * kR256Rows, per_cu)), dim3(kBlock),
                  s, a);
}

template <int CB>
hipError_t run_rdq256_cb(const DequantArgs &a, hipStream_t s) {
    static const int per_cu = resident_blocks(k_residual_dequantize_mfma256<CB>);
    return launch(k_residual_dequantize_mfma256<CB>, dim3(grid_for(a.n, kWaves * kR256Rows, per_cu)),
                  dim3(kBlock), s, a);
}

hipError_t run_res256(int cb, const QuantArgs &a, hipStream_t s) {
    switch (cb) {
    case 1: return run_res256_cb<1>(a, s);
    case 2: return run_res256_cb<2>(a, s);
    case 3: return run_res256_cb<3>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t quant_d(bool f16, int bits, Kind kind, const QuantArgs &a, hipStream_t s) {
    constexpr int E = D / lanes_per_vec(D);
    switch (kind) {
    case kMse:
        if (D == 128 && f16 && bits == 4 && hadamard_on_mfma()) return launch_quantize_kv128(a, s);
        // one 32-bit code word per lane-group (G = 32 / bits); 3-bit codes: contiguous runs
        switch (bits) {
        case 1: return f16 ? run_q<D, 32, true, 1, kMse>(a, s) : run_q<D, 32, false, 1, kMse>(a, s);
        case 2: return f16 ? run_q<D, 16, true, 2, kMse>(a, s) : run_q<D, 16, false, 2, kMse>(a, s);
        case 3: return f16 ? run_q<D, E, true, 3, kMse>(a, s) : run_q<D, E, false, 3, kMse>(a, s);
        case 4: return f16 ? run_q<D, 8, true, 4, kMse>(a, s) : run_q<D, 8, false, 4, kMse>(a, s);
        }
        break;
    case kDriveBiased:
        return f16 ? run_q<D, E, true, 1, kDriveBiased>(a, s) : run_q<D, E, false, 1, kDriveBiased>(a, s);
    case kDriveUnbiased:
        return f16 ? run_q<D, E, true, 1, kDriveUnbiased>(a, s)
                   : run_q<D, E, false, 1, kDriveUnbiased>(a, s);
    case kResidual:
        if (D == 256 && f16 && hadamard_on_mfma()) return run_res256(bits - 1, a, s);
        switch (bits) {
        case 2: return f16 ? run_q<D, E, true, 2, kResidual>(a, s) : run_q<D, E, false, 2, kResidual>(a, s);
        case 3: return f16 ? run_q<D, E, true, 3, kResidual>(a, s) : run_q<D, E, false, 3, kResidual>(a, s);
        case 4: return f16 ? run_q<D, E, true, 4, kResidual>(a, s) : run_q<D, E, false, 4, kResidual>(a, s);
        }
        break;
    case kEden:
        switch (bits) {
        case 1: return f16 ? run_q<D, E, true, 1, kEden>(a, s) : run_q<D, E, false, 1, kEden>(a, s);
        case 2: return f16 ? run_q<D, E, true, 2, kEden>(a, s) : run_q<D, E, false, 2, kEden>(a, s);
        case 3: return f16 ? run_q<D, E, true, 3, kEden>(a, s) : run_q<D, E, false, 3, kEden>(a, s);
        case 4: return f16 ? run_q<D, E, true, 4, kEden>(a, s) : run_q<D, E, false, 4, kEden>(a, s);
        }
        break;
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t dequant_d(bool f16, int bits, Kind kind, const DequantArgs &a, hipStream_t s) {
    constexpr int E = D / lanes_per_vec(D);
    switch (kind) {
    case kMse:
        if (D == 128 && f16 && bits == 4 && hadamard_on_mfma()) return launch_dequantize_kv128(a, s);
        switch (bits) {
        case 1: return f16 ? run_dq<D, 32, true, 1, kMse>(a, s) : run_dq<D, 32, false, 1, kMse>(a, s);
        case 2: return f16 ? run_dq<D, 16, true, 2, kMse>(a, s) : run_dq<D, 16, false, 2, kMse>(a, s);
        case 3: return f16 ? run_dq<D, E, true, 3, kMse>(a, s) : run_dq<D, E, false, 3, kMse>(a, s);
        case 4: return f16 ? run_dq<D, 8, true, 4, kMse>(a, s) : run_dq<D, 8, false, 4, kMse>(a, s);
        }
        break;
    case kDriveBiased:
    case kDriveUnbiased:
        return f16 ? run_dq<D, E, true, 1, kDriveBiased>(a, s) : run_dq<D, E, false, 1, kDriveBiased>(a, s);
    case kResidual:
        if (D == 256 && f16 && hadamard_on_mfma()) {
            if (bits == 2) return run_rdq256_cb<1>(a, s);
            if (bits == 3) return run_rdq256_cb<2>(a, s);
        }
        switch (bits) {
        case 2: return f16 ? run_dq<D, E, true, 2, kResidual>(a, s) : run_dq<D, E, false, 2, kResidual>(a, s);
        case 3: return f16 ? run_dq<D, E, true, 3, kResidual>(a, s) : run_dq<D, E, false, 3, kResidual>(a, s);
        case 4: return f16 ? run_dq<D, E, true, 4, kResidual>(a, s) : run_dq<D, E, false, 4, kResidual>(a, s);
        }
        break;
    case kEden:  // EDEN codes decode as MSE codes (the caller passes kMse)
        break;
    }
    return hipErrorInvalidValue;
}

template <int D, int BITS, bool RES>
hipError_t run_score(const ScoreArgs &a, hipStream_t s) {
    const int64_t tiles = (a.n + 31) / 32;
    int64_t blocks = (tiles + kWaves - 1) / kWaves;
    const int64_t cap = (int64_t)device_cu_count() * 2;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    return launch(k_score<D, BITS, RES>, dim3((int)blocks), dim3(kBlock), s, a);
}

template <int D, int BITS, bool RES, bool EXACT>
hipError_t run_score_mfma(const ScoreArgs &a, hipStream_t s) {
    static const int per_cu = resident_blocks(k_score_mfma<D, BITS, RES, EXACT>);
    // wave items: (pair of key tiles, query half); a block serves one half
    const int rh = a.m > 32 ? 2 : 1;
    const int64_t items = ((a.n + 32 * kScoreTK - 1) / (32 * kScoreTK)) * rh;
    // two blocks per CU: each block rotates its query half once, and fewer,
    // longer blocks repeat that less (sign codes: 13.5 -> 12.9 us on 131072
    // keys; MSE and residual codes unchanged)
    int blocks = capped_grid(items, kWaves, per_cu, 2);
    if (rh == 2) blocks = (blocks + 15) / 16 * 16;  // the kernel pairs blocks b and b + 8
    return launch(k_score_mfma<D, BITS, RES, EXACT>, dim3(blocks), dim3(kBlock), s, a);
}

template <int D, int BITS, bool RES>
hipError_t run_score_wide(const ScoreArgs &a, hipStream_t s) {
    static const int per_cu = resident_blocks(k_score_wide<D, BITS, RES>);
    constexpr int QG = wide_score_group<D>();
    const int64_t G = (a.m + QG - 1) / QG;
    const int64_t tiles = (a.n + 31) / 32;
    // tile-blocks (kWaves tiles per round each), a multiple of 8 so every
    // group of a tile-block sits on the same XCD; at most what is resident
    int64_t tbs = (tiles + kWaves - 1) / kWaves;
    const int64_t cap_tbs = (int64_t)device_cu_count() * min(per_cu, 2) / G;
    if (tbs > cap_tbs) tbs = cap_tbs;
    tbs = (tbs + 7) / 8 * 8;
    if (tbs < 8) tbs = 8;
    return launch(k_score_wide<D, BITS, RES>, dim3((unsigned)(tbs * G)), dim3(kBlock), s, a);
}

template <int D>
hipError_t score_wide_d(int bits, bool residual, const ScoreArgs &a, hipStream_t s) {
    if (residual) {
        switch (bits) {
        case 1: return run_score_wide<D, 1, true>(a, s);
        case 2: return run_score_wide<D, 2, true>(a, s);
        case 3: return run_score_wide<D, 3, true>(a, s);
        }
        return hipErrorInvalidValue;
    }
    switch (bits) {
    case 1: return run_score_wide<D, 1, false>(a, s);
    case 2: return run_score_wide<D, 2, false>(a, s);
    case 3: return run_score_wide<D, 3, false>(a, s);
    case 4: return run_score_wide<D, 4, false>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t score_mfma_d(int bits, bool residual, const ScoreArgs &a, hipStream_t s) {
    if (residual) {
        switch (bits) {
        case 1: return run_score_mfma<D, 1, true, false>(a, s);
        case 2: return run_score_mfma<D, 2, true, false>(a, s);
        case 3: return run_score_mfma<D, 3, true, false>(a, s);
        }
        return hipErrorInvalidValue;
    }
    switch (bits) {
    case 1: return a.exact ? run_score_mfma<D, 1, false, true>(a, s) : run_score_mfma<D, 1, false, false>(a, s);
    case 2: return run_score_mfma<D, 2, false, false>(a, s);
    case 3: return run_score_mfma<D, 3, false, false>(a, s);
    case 4: return run_score_mfma<D, 4, false, false>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t score_d(int bits, bool residual, const ScoreArgs &a, hipStream_t s) {
    if constexpr (D == 128) {
        if (hadamard_on_mfma()) return score_mfma_d<D>(bits, residual, a, s);
    }
    if (residual) {
        switch (bits) {
        case 1: return run_score<D, 1, true>(a, s);
        case 2: return run_score<D, 2, true>(a, s);
        case 3: return run_score<D, 3, true>(a, s);
        }
        return hipErrorInvalidValue;
    }
    switch (bits) {
    case 1: return run_score<D, 1, false>(a, s);
    case 2: return run_score<D, 2, false>(a, s);
    case 3: return run_score<D, 3, false>(a, s);
    case 4: return run_score<D, 4, false>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_quantize(int d, bool f16, int bits, Kind kind, const QuantArgs &a, hipStream_t s) {
    switch (d) {
    case 16: return launch_quantize_d16(f16, bits, kind, a, s);
    case 32: return quant_d<32>(f16, bits, kind, a, s);
    case 64: return quant_d<64>(f16, bits, kind, a, s);
    case 128: return quant_d<128>(f16, bits, kind, a, s);
    case 256: return quant_d<256>(f16, bits, kind, a, s);
    case 512: return quant_d<512>(f16, bits, kind, a, s);
    case 1024: return quant_d<1024>(f16, bits, kind, a, s);
    case 2048: return quant_d<2048>(f16, bits, kind, a, s);
    case 4096: return quant_d<4096>(f16, bits, kind, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_dequantize(int d, bool f16out, int bits, Kind kind, const DequantArgs &a, hipStream_t s) {
    switch (d) {
    case 16: return launch_dequantize_d16(f16out, bits, kind, a, s);
    case 32: return dequant_d<32>(f16out, bits, kind, a, s);
    case 64: return dequant_d<64>(f16out, bits, kind, a, s);
    case 128: return dequant_d<128>(f16out, bits, kind, a, s);
    case 256: return dequant_d<256>(f16out, bits, kind, a, s);
    case 512: return dequant_d<512>(f16out, bits, kind, a, s);
    case 1024: return dequant_d<1024>(f16out, bits, kind, a, s);
    case 2048: return dequant_d<2048>(f16out, bits, kind, a, s);
    case 4096: return dequant_d<4096>(f16out, bits, kind, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_score(int d, int bits, bool residual, const ScoreArgs &a, hipStream_t s) {
    switch (d) {
    case 16: return launch_score_d16(bits, residual, a, s);
    case 32: return score_d<32>(bits, residual, a, s);
    case 64: return score_d<64>(bits, residual, a, s);
    case 128: return score_d<128>(bits, residual, a, s);
    case 256: return score_d<256>(bits, residual, a, s);
    case 512: return score_wide_d<512>(bits, residual, a, s);
    case 1024: return score_wide_d<1024>(bits, residual, a, s);
    case 2048: return score_wide_d<2048>(bits, residual, a, s);
    case 4096: return score_wide_d<4096>(bits, residual, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace rht
