// rht_attn.hip -- attention of a few queries over MSE-coded keys and values
// (d = 128, 4-bit codes), computed in the rotated domains.
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
// 2^-22 relative) and summing hi*hi + hi*lo + lo*hi in the fp32 accumulator.
//   logits:  C[key][query] = sum_k A[key][k] B[k][query], A = code levels of
//            16 keys (hi/lo from a 256-entry byte table), B = H D_k q scaled by
//            a power of two into fp16 range.
//   values:  z^T[coord][query] += sum_key Cv^T[coord][key] P[key][query],
//            P = p_j ||v_j|| times a running power of two; the accumulator
//            layout of the logits tiles is exactly the B layout P needs.
// Lane layout of the 16x16x32 instruction (lane l, g = l / 16): A holds
// A[l % 16][8 g + t], B holds B[8 g + t][l % 16], C holds C[4 g + r][l % 16].
#include "rht_device.h"

namespace rht {
namespace {

constexpr int kAD = 128;           // coordinates per vector
constexpr int kACodeBytes = 64;    // 4-bit codes per row
constexpr int kVRow = 80;          // LDS row stride of a staged value tile (bank spread)

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

// 2^e for e <= 0, flushed to 0 below the normal range.
__device__ __forceinline__ float pow2i_down(int e) { return e < -126 ? 0.0f : pow2i(e); }

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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

// Clamped fp32 load of element idx of a row of n (n >= 1).
__device__ __forceinline__ float load_clamped(const float *p, int64_t idx, int64_t n) {
    return p[idx < n ? idx : n - 1];
}

// Global loads of one 32-key tile for a lane: K code bytes 16g..16g+15 of keys
// key0 + l%16 and key0 + 16 + l%16; the lane's two 16-byte pieces of the value
// tile (chunks l and 64 + l of the 32 x 64-byte tile); the key and value norms
// of the keys this lane's accumulator rows hold (4g + r and 16 + 4g + r).
struct TileRegs {
    u32x4_t k0, k1, v0, v1;
    float kn[8], vn[8];
};

__device__ __forceinline__ void load_tile(const AttnArgs &a, const uint8_t *kc, const uint8_t *vc,
                                          const float *kn, const float *vn, int64_t key0, uint32_t lane,
                                          TileRegs &t) {
    const uint32_t j = lane & 15u, g = lane >> 4;
    const int64_t n = a.n;
    auto row = [n](int64_t r) { return r < n ? r : n - 1; };
    t.k0 = *reinterpret_cast<const u32x4_t *>(kc + row(key0 + j) * kACodeBytes + 16 * g);
    t.k1 = *reinterpret_cast<const u32x4_t *>(kc + row(key0 + 16 + j) * kACodeBytes + 16 * g);
    t.v0 = *reinterpret_cast<const u32x4_t *>(vc + row(key0 + lane / 4) * kACodeBytes + 16 * (lane % 4));
    t.v1 = *reinterpret_cast<const u32x4_t *>(vc + row(key0 + 16 + lane / 4) * kACodeBytes + 16 * (lane % 4));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        t.kn[r] = load_clamped(kn, key0 + 4 * g + r, n);
        t.kn[4 + r] = load_clamped(kn, key0 + 16 + 4 * g + r, n);
        t.vn[r] = load_clamped(vn, key0 + 4 * g + r, n);
        t.vn[4 + r] = load_clamped(vn, key0 + 16 + 4 * g + r, n);
    }
}

// Logits of 16 keys (one 16-byte code piece per lane) against the queries.
__device__ __forceinline__ floatx4 key_logits(const uint2 *tab, u32x4_t kc, const u32x4_t (&bh)[4],
                                              const u32x4_t (&bl)[4]) {
    floatx4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const uint32_t w = kc[ks];
        const uint2 e0 = tab[w & 0xFFu], e1 = tab[(w >> 8) & 0xFFu];
        const uint2 e2 = tab[(w >> 16) & 0xFFu], e3 = tab[w >> 24];
        const u32x4_t ah = {e0.x, e1.x, e2.x, e3.x}, al = {e0.y, e1.y, e2.y, e3.y};
        c = mfma1632(ah, bh[ks], c);
        c = mfma1632(ah, bl[ks], c);
        c = mfma1632(al, bh[ks], c);
    }
    return c;
}

__global__ __launch_bounds__(kBlock) void k_attn_partial(const AttnArgs a) {
    __shared__ uint2 tab[256];
    __shared__ float qbuf[kWaves][16][kAD];
    __shared__ __attribute__((aligned(16))) uint8_t vbuf[kWaves][32 * kVRow];
    {
        const uint32_t v = threadIdx.x;
        tab[v] = split2(a.lev[v & 15u], a.lev[v >> 4]);
    }
    __syncthreads();

    const uint32_t lane = lane_id(), wave = threadIdx.x >> 6, j = lane & 15u, g = lane >> 4;
    const int64_t gw = (int64_t)blockIdx.x * kWaves + wave;
    if (gw >= a.heads * a.chunks) return;  // whole wave; no block barrier follows
    const int64_t head = gw / a.chunks;
    const int chunk = (int)(gw % a.chunks);
    const int64_t tiles = (a.n + 31) / 32;
    const int64_t t_begin = tiles * chunk / a.chunks, t_end = tiles * (chunk + 1) / a.chunks;

    // --- queries: q~ = H D_k q, scaled by 2^(14 - e) into fp16 range
    float qscale_mine = 1.0f;  // power of two applied to query j
    for (int i = 0; i < 16; ++i) {
        float v0 = 0.0f, v1 = 0.0f;
        if (i < a.m) {
            const float2 qv = reinterpret_cast<const float2 *>(a.q + (head * a.m + i) * kAD)[lane];
            const uint32_t sb = a.dsign_k[lane >> 4] >> ((2 * lane) & 31);
            v0 = (sb & 1u) ? -qv.x : qv.x;
            v1 = (sb & 2u) ? -qv.y : qv.y;
            fwht128_pairs(v0, v1, lane);
        }
        const float mx = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
        const float sc = mx > 0.0f ? pow2i(min(14 - exponent_above(mx), 126)) : 1.0f;
        if ((uint32_t)i == j) qscale_mine = sc;
        qbuf[wave][i][2 * lane] = v0 * sc;
        qbuf[wave][i][2 * lane + 1] = v1 * sc;
    }
    // B operand of the logits: B[k][query j] for K step ks, k = 8g + t <-> coordinate 32g + 8ks + t
    u32x4_t bh[4], bl[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        uint32_t h[4], l[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int c = 32 * g + 8 * ks + 2 * w;
            const uint2 s = split2(qbuf[wave][j][c], qbuf[wave][j][c + 1]);
            h[w] = s.x;
            l[w] = s.y;
        }
        bh[ks] = u32x4_t{h[0], h[1], h[2], h[3]};
        bl[ks] = u32x4_t{l[0], l[1], l[2], l[3]};
    }
    // logits in base-2 units: s = C * ||k|| * fq
    const float fq = a.scale * 1.4426950408889634f / ((float)kAD * qscale_mine);

    const uint8_t *kc = a.kc + head * a.n * kACodeBytes;
    const uint8_t *vc = a.vc + head * a.n * kACodeBytes;
    const float *kn = a.kn + head * a.n;
    const float *vn = a.vn + head * a.n;
    uint8_t *vb = vbuf[wave];

    float M = -INFINITY, l = 0.0f;
    int ev = -100;  // value scale exponent: P = p ||v|| 2^(14 - ev)
    floatx4 ze[4], zo[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        ze[p] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        zo[p] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    TileRegs nxt;
    if (t_begin < t_end) load_tile(a, kc, vc, kn, vn, t_begin * 32, lane, nxt);
    for (int64_t tile = t_begin; tile < t_end; ++tile) {
        const int64_t key0 = tile * 32;
        const TileRegs cur = nxt;
        // stage the value codes: key r at vb + r * kVRow
        *reinterpret_cast<u32x4_t *>(vb + (lane / 4) * kVRow + 16 * (lane % 4)) = cur.v0;
        *reinterpret_cast<u32x4_t *>(vb + (16 + lane / 4) * kVRow + 16 * (lane % 4)) = cur.v1;
        if (tile + 1 < t_end) load_tile(a, kc, vc, kn, vn, key0 + 32, lane, nxt);

        // logits: rows 4g + r of tile 0 are keys 4g + r, of tile 1 keys 16 + 4g + r
        const floatx4 c0 = key_logits(tab, cur.k0, bh, bl);
        const floatx4 c1 = key_logits(tab, cur.k1, bh, bl);
        float s[8], vmax = 0.0f, smax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int64_t key = key0 + (r < 4 ? 4 * g + r : 16 + 4 * g + (r - 4));
            const float cv = r < 4 ? c0[r] : c1[r - 4];
            s[r] = key < a.n ? cv * cur.kn[r] * fq : -INFINITY;
            smax = fmaxf(smax, s[r]);
            if (key < a.n) vmax = fmaxf(vmax, cur.vn[r]);
        }
        smax = fmaxf(smax, __shfl_xor(smax, 16));
        smax = fmaxf(smax, __shfl_xor(smax, 32));
        vmax = fmaxf(vmax, __shfl_xor(vmax, 16));
        vmax = fmaxf(vmax, __shfl_xor(vmax, 32));
        const float Mn = fmaxf(M, smax);
        const int evn = vmax > 0.0f ? max(ev, exponent_above(vmax)) : ev;
        // rescale the running sums to the new max and value scale
        const float alpha = __builtin_amdgcn_exp2f(M - Mn);
        const float rz = alpha * pow2i_down(ev - evn);
        M = Mn;
        ev = evn;
        l *= alpha;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            ze[p] *= rz;
            zo[p] *= rz;
        }
        const float vs = pow2i(14 - ev);
        float P[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float pr = __builtin_amdgcn_exp2f(s[r] - M);
            l += pr;
            P[r] = pr * cur.vn[r] * vs;
        }
        // B operand of the value product: k = 8g + t <-> key (t < 4 ? 4g + t : 16 + 4g + t - 4)
        u32x4_t ph, pl;
        {
            const uint2 s0 = split2(P[0], P[1]), s1 = split2(P[2], P[3]);
            const uint2 s2 = split2(P[4], P[5]), s3 = split2(P[6], P[7]);
            ph = u32x4_t{s0.x, s1.x, s2.x, s3.x};
            pl = u32x4_t{s0.y, s1.y, s2.y, s3.y};
        }
        // A operand: row = coordinate 32p + 2 (l % 16) + e, k = 8g + t <-> the key above;
        // code byte 16p + l % 16 of that key holds both coordinates of the pair.
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint2 e[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const uint32_t key = t < 4 ? 4 * g + t : 16 + 4 * g + (t - 4);
                e[t] = tab[vb[key * kVRow + 16 * p + j]];
            }
            u32x4_t aeh, aol, ael, aoh;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // low halves (even coordinate) and high halves (odd) of keys 2w, 2w+1
                aeh[w] = __builtin_amdgcn_perm(e[2 * w + 1].x, e[2 * w].x, 0x05040100u);
                aoh[w] = __builtin_amdgcn_perm(e[2 * w + 1].x, e[2 * w].x, 0x07060302u);
                ael[w] = __builtin_amdgcn_perm(e[2 * w + 1].y, e[2 * w].y, 0x05040100u);
                aol[w] = __builtin_amdgcn_perm(e[2 * w + 1].y, e[2 * w].y, 0x07060302u);
            }
            ze[p] = mfma1632(aeh, ph, ze[p]);
            ze[p] = mfma1632(aeh, pl, ze[p]);
            ze[p] = mfma1632(ael, ph, ze[p]);
            zo[p] = mfma1632(aoh, ph, zo[p]);
            zo[p] = mfma1632(aoh, pl, zo[p]);
            zo[p] = mfma1632(aol, ph, zo[p]);
        }
    }
    // l: each lane group g summed its own keys
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if ((int)j < a.m && t_begin < t_end) {
        float *rec = a.ws + ((head * a.chunks + chunk) * a.m + j) * kAttnRecord;
        // accumulator row 4g + r of pair p is coordinate 32p + 8g + 2r (+1 for the odd tile)
        const float zs = pow2i(ev - 14) * (1.0f / (float)kAD);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            float4 lo, hi;
            lo.x = ze[p][0] * zs; lo.y = zo[p][0] * zs; lo.z = ze[p][1] * zs; lo.w = zo[p][1] * zs;
            hi.x = ze[p][2] * zs; hi.y = zo[p][2] * zs; hi.z = ze[p][3] * zs; hi.w = zo[p][3] * zs;
            reinterpret_cast<float4 *>(rec + 32 * p + 8 * g)[0] = lo;
            reinterpret_cast<float4 *>(rec + 32 * p + 8 * g)[1] = hi;
        }
        if (g == 0) {
            rec[kAD] = M;
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
    float M = -INFINITY;
    for (int c = 0; c < a.chunks; ++c) M = fmaxf(M, rec0[c * step + kAD]);
    float z0 = 0.0f, z1 = 0.0f, l = 0.0f;
    for (int c = 0; c < a.chunks; ++c) {
        const float *rec = rec0 + c * step;
        const float w = __builtin_amdgcn_exp2f(rec[kAD] - M);
        const float2 zv = reinterpret_cast<const float2 *>(rec)[lane];
        z0 = fmaf(w, zv.x, z0);
        z1 = fmaf(w, zv.y, z1);
        l = fmaf(w, rec[kAD + 1], l);
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

hipError_t launch_attention(const AttnArgs &a, hipStream_t s) {
    const int64_t waves = a.heads * a.chunks;
    hipLaunchKernelGGL(k_attn_partial, dim3((unsigned)((waves + kWaves - 1) / kWaves)), dim3(kBlock), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = a.heads * a.m;
    hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)((rows + kWaves - 1) / kWaves)), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace rht
