// stream_ceiling.hip -- trivial streaming kernels with the exact HBM traffic
// of the d = 128, fp16, 4-bit encoder and decoder, used by the benchmark as
// the achievable ceiling for those shapes on this GPU.  Not part of librht.
//
//   encode shape: read 256 B (an fp16 row), write 64 B (codes) + 4 B (scale)
//   decode shape: read 64 B + 4 B, write 256 B
//
// Each wavefront moves 16 rows per step with 16-byte accesses, every access
// instruction covering whole contiguous KiB pieces (lane l, instruction k:
// chunk 64 k + l), non-temporal loads and stores like the library's streaming
// kernels.  The only arithmetic is an XOR fold, so nothing but the memory
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

}  // extern "C"
