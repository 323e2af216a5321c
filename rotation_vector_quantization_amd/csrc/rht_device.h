// rht_device.h -- device-side pieces shared by the kernel sources: launch
// shape, vector types, the fp16 dot product, the nearest-level table and grid
// sizing.  Included by .hip files only.
#pragma once

#include "rht_internal.h"

namespace rht {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

__host__ __device__ constexpr int lanes_per_vec(int d) { return d >= 4096 ? 64 : d / 32; }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63u; }

// Word 3 of a CDNA raw buffer resource: data format 32 bits, no swizzle, no
// index stride (the offsets are byte offsets, range-checked against the
// resource's size: a load past it returns zeros).
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                  false);
}

// Nearest-level table for y16 = 16 * y.  Cell k holds the y16 values with
// round(y16 + OFF) == k; its entry is (scaled threshold that may lie in the
// cell or +inf, code at the cell's low end).  Each entry is built for the
// widened window [k - OFF - 0.75, k - OFF + 1.25), so it stays right whatever
// the rounding of the index; windows are 2 wide and scaled thresholds are at
// least 4 apart (16 x the smallest N(0,1) Lloyd-Max gap), so a window holds at
// most one threshold.
template <int NCELL, int OFF>
__device__ __forceinline__ void build_lut(uint2 *lut, const float *thr, int nthr) {
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
        lut[k] = make_uint2(__builtin_bit_cast(uint32_t, t_in), base);
    }
}

// |y16| <= 16 sqrt(d) (|(H D x)_i| <= ||x||_1 <= sqrt(d) ||x||), so for d <= 128
// a 512-cell table centred on 0 needs no clamp; larger d clamp into 256 cells.
template <int D>
struct Lut {
    static constexpr bool kClamp = D > 128;
    static constexpr int kCells = kClamp ? 256 : 512;
    static constexpr int kOff = kClamp ? 40 : 256;
};

template <int D>
__device__ __forceinline__ uint32_t nearest_code(const uint2 *lut, float y16) {
    // adding 2^23 + OFF leaves round(y16 + OFF) in the low mantissa bits
    int b = __builtin_bit_cast(int, y16 + (8388608.0f + (float)Lut<D>::kOff));
    if constexpr (Lut<D>::kClamp) b = min(max(b, 0x4B000000), 0x4B000000 + Lut<D>::kCells - 1);
    const uint2 e = lut[b - 0x4B000000];
    return e.y + (y16 >= __builtin_bit_cast(float, e.x) ? 1u : 0u);
}

// Queue kernel(args...) on `s` and return the status of this launch itself:
// hipLaunchKernel reports the launch it was handed, where hipGetLastError
// would also return (and clear) an error that an earlier, unrelated HIP call
// on this thread left behind.
template <typename... P, typename... A>
inline hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s, const A &...args) {
    static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
    void *argv[] = {const_cast<void *>(static_cast<const void *>(&args))...};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, 0, s);
}

// ---------------------------------------------------------------------------
// Grid sizing.  Grids are sized to what is resident at once (CUs x
// blocks per CU from the occupancy calculator), so every block of the
// grid-stride loop gets the same share and there is no partial last wave.
template <typename K>
int resident_blocks(K kernel) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    return per_cu;
}

// Fewer, longer-lived blocks measured faster than a full-occupancy grid: the
// streaming loads are prefetched one vector ahead in every wave, and HBM
// write throughput drops with many concurrent writers.
constexpr int kDefaultBlocksPerCU = 3;

inline int grid_for(int64_t n, int vpb, int per_cu) {
    if (per_cu > kDefaultBlocksPerCU) per_cu = kDefaultBlocksPerCU;
    const int64_t want = (n + vpb - 1) / vpb;
    const int64_t cap = (int64_t)device_cu_count() * per_cu;
    return (int)(want < cap ? (want > 0 ? want : 1) : cap);
}

}  // namespace
}  // namespace rht
