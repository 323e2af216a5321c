// stream_ceiling.hip -- trivial streaming kernels with the exact HBM traffic
// of the d = 128, fp16, 4-bit encoder and decoder and of 4-bit scoring, used by the benchmark as
// the achievable ceiling for those shapes on this GPU.  Not part of librht.
//
//   encode shape: read 256 B (an fp16 row), write 64 B (codes) + 4 B (scale)
//   decode shape: read 64 B + 4 B, write 256 B
//   score shape:  read 64 B (4-bit codes of a d = 128 key) + 4 B (norm), write
//                 m fp32 logits, one in each of m rows of n keys
//
// Each wavefront moves 16 rows per step (KV shapes) with 16-byte accesses, every access
// instruction covering whole contiguous KiB pieces (lane l, instruction k:
// chunk 64 k + l), non-temporal loads and stores like the library's streaming
// kernels (the score shape: 64 keys per step, 4-byte logit stores as the scorer
// makes them).  The only arithmetic is an XOR fold, so nothing but the memory
// system sets the time.  Grids are CUs x blocks-per-CU, grid-stride loops; the
// next step's loads are issued before the current step's stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

__global__ __launch_bounds__(kBlock) void k_encode_shape(const u32x4_t *__restrict__ x, u32x4_t *__restrict__ codes,
                                                          float *__restrict__ scale, int64_t groups) {
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    int64_t g = (int64_t)blockIdx.x * kWaves + wave;
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    if (g >= groups) return;
    // 16 rows x 16 chunks of input per group, 16 x 4 chunks of codes, 16 scales
    const u32x4_t *src = x + g * 256;
    u32x4_t a0 = __builtin_nontemporal_load(src + lane), a1 = __builtin_nontemporal_load(src + 64 + lane);
    u32x4_t a2 = __builtin_nontemporal_load(src + 128 + lane), a3 = __builtin_nontemporal_load(src + 192 + lane);
    for (;;) {
        const int64_t next = g + stride;
        const u32x4_t o = a0 ^ a1 ^ a2 ^ a3;
        if (next < groups) {
            const u32x4_t *s2 = x + next * 256;
            a0 = __builtin_nontemporal_load(s2 + lane);
            a1 = __builtin_nontemporal_load(s2 + 64 + lane);
            a2 = __builtin_nontemporal_load(s2 + 128 + lane);
            a3 = __builtin_nontemporal_load(s2 + 192 + lane);
        }
        __builtin_nontemporal_store(o, codes + g * 64 + lane);
        if (lane < 16) __builtin_nontemporal_store(__builtin_bit_cast(float, o.x ^ o.w), scale + g * 16 + lane);
        g = next;
        if (g >= groups) break;
    }
}

__global__ __launch_bounds__(kBlock) void k_decode_shape(const u32x4_t *__restrict__ codes,
                                                          const float *__restrict__ scale, u32x4_t *__restrict__ y,
                                                          int64_t groups) {
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    int64_t g = (int64_t)blockIdx.x * kWaves + wave;
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    if (g >= groups) return;
    u32x4_t c = __builtin_nontemporal_load(codes + g * 64 + lane);
    float s = lane < 16 ? __builtin_nontemporal_load(scale + g * 16 + lane) : 0.0f;
    for (;;) {
        const int64_t next = g + stride;
        const uint32_t sv = __builtin_bit_cast(uint32_t, __shfl(s, (int)(lane / 4)));
        const u32x4_t base = c ^ sv;
        if (next < groups) {
            c = __builtin_nontemporal_load(codes + next * 64 + lane);
            s = lane < 16 ? __builtin_nontemporal_load(scale + next * 16 + lane) : 0.0f;
        }
        u32x4_t *dst = y + g * 256;
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k) __builtin_nontemporal_store(base ^ k, dst + 64 * k + lane);
        g = next;
        if (g >= groups) break;
    }
}

// Score shape, in the scorer's own order: a block serves one half of the m
// <= 64 logit rows (32 each); with two halves, blocks b and b + 8 (which the
// GPU places on the same XCD) take the same keys, one half each, so the
// second read of a key range can hit that XCD's L2.  A wave step is 64 keys
// (4 KiB of codes, 64 norms); store instruction (r, t) writes logit row
// 32 half + 8 (r / 4) + 4 h + r % 4 (lane half h) at keys 32 t + lane % 32, so
// each instruction writes two 128-byte runs.
__global__ __launch_bounds__(kBlock) void k_score_shape(const u32x4_t *__restrict__ codes,
                                                         const float *__restrict__ norms, float *__restrict__ logits,
                                                         int64_t n, int m) {
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6, i = lane & 31u, h = lane >> 5;
    const int RH = m > 32 ? 2 : 1;
    const uint32_t b = blockIdx.x;
    const int rh = RH == 2 ? (int)((b >> 3) & 1u) : 0;
    const uint32_t ib = RH == 2 ? ((b >> 4) << 3) + (b & 7u) : b;
    const int64_t groups = n / 64;
    int64_t g = (int64_t)ib * kWaves + wave;
    const int64_t stride = (int64_t)(gridDim.x / RH) * kWaves;
    if (g >= groups) return;
    const u32x4_t *src = codes + g * 256;
    u32x4_t a0 = __builtin_nontemporal_load(src + lane), a1 = __builtin_nontemporal_load(src + 64 + lane);
    u32x4_t a2 = __builtin_nontemporal_load(src + 128 + lane), a3 = __builtin_nontemporal_load(src + 192 + lane);
    float s = __builtin_nontemporal_load(norms + g * 64 + lane);
    for (;;) {
        const int64_t next = g + stride;
        const u32x4_t o = a0 ^ a1 ^ a2 ^ a3;
        const uint32_t f = o.x ^ o.y ^ o.z ^ o.w ^ __builtin_bit_cast(uint32_t, s);
        if (next < groups) {
            const u32x4_t *s2 = codes + next * 256;
            a0 = __builtin_nontemporal_load(s2 + lane);
            a1 = __builtin_nontemporal_load(s2 + 64 + lane);
            a2 = __builtin_nontemporal_load(s2 + 128 + lane);
            a3 = __builtin_nontemporal_load(s2 + 192 + lane);
            s = __builtin_nontemporal_load(norms + next * 64 + lane);
        }
        for (int r = 0; r < 16; ++r) {
            const int q = 32 * rh + 8 * (r / 4) + 4 * (int)h + r % 4;
            if (q < m) {
                float *row = logits + (int64_t)q * n + g * 64 + i;
                __builtin_nontemporal_store(__builtin_bit_cast(float, f ^ (uint32_t)r), row);
                __builtin_nontemporal_store(__builtin_bit_cast(float, f + (uint32_t)r), row + 32);
            }
        }
        g = next;
        if (g >= groups) break;
    }
}

int cu_count() {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return -1;
    return v;
}

}  // namespace

extern "C" {

// n rows (a multiple of 16), blocks_per_cu in [1, 16]; device pointers, 16-byte
// aligned; queued on `stream`.  Returns 0, -1 for bad arguments, or the HIP
// error code of the launch.
int ceiling_encode_shape(const void *x, void *codes, float *scale, int64_t n, int blocks_per_cu, void *stream) {
    if (n <= 0 || n % 16 || blocks_per_cu < 1 || blocks_per_cu > 16 || !x || !codes || !scale) return -1;
    const int cus = cu_count();
    if (cus <= 0) return -1;
    const int64_t groups = n / 16;
    void *argv[] = {(void *)&x, (void *)&codes, (void *)&scale, (void *)&groups};
    return (int)hipLaunchKernel((const void *)k_encode_shape, dim3(cus * blocks_per_cu), dim3(kBlock), argv, 0,
                                (hipStream_t)stream);
}

int ceiling_decode_shape(const void *codes, const float *scale, void *y, int64_t n, int blocks_per_cu, void *stream) {
    if (n <= 0 || n % 16 || blocks_per_cu < 1 || blocks_per_cu > 16 || !codes || !scale || !y) return -1;
    const int cus = cu_count();
    if (cus <= 0) return -1;
    const int64_t groups = n / 16;
    void *argv[] = {(void *)&codes, (void *)&scale, (void *)&y, (void *)&groups};
    return (int)hipLaunchKernel((const void *)k_decode_shape, dim3(cus * blocks_per_cu), dim3(kBlock), argv, 0,
                                (hipStream_t)stream);
}

// n keys (a multiple of 64), m logit rows (1 to 64),
// blocks_per_cu in [1, 16]; logits is [m][n] fp32.  Same conventions as above.
int ceiling_score_shape(const void *codes, const float *norms, float *logits, int64_t n, int m, int blocks_per_cu,
                        void *stream) {
    if (n <= 0 || n % 64 || m < 1 || m > 64 || blocks_per_cu < 1 || blocks_per_cu > 16 || !codes ||
        !norms || !logits)
        return -1;
    const int cus = cu_count();
    if (cus <= 0) return -1;
    // with two row halves the kernel pairs blocks b and b + 8: a multiple of 16 blocks
    const int blocks = m > 32 ? (cus * blocks_per_cu + 15) / 16 * 16 : cus * blocks_per_cu;
    void *argv[] = {(void *)&codes, (void *)&norms, (void *)&logits, (void *)&n, (void *)&m};
    return (int)hipLaunchKernel((const void *)k_score_shape, dim3(blocks), dim3(kBlock), argv, 0,
                                (hipStream_t)stream);
}

}  // extern "C"
