// Device-side helpers shared by the gfx950 kernels of libmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Host side: raises `kernel`'s dynamic-LDS limit to `bytes` on the current
// device (hipFuncSetAttribute acts on the device current at the call), once
// per device and size. `done` holds, per device, the largest limit set so
// far; give each kernel instantiation an array of its own.
constexpr int kMaxDevices = 64;
inline hipError_t ensure_dynamic_lds(const void* kernel, int bytes, std::atomic<int>* done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices && done[dev].load(std::memory_order_acquire) >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && dev >= 0 && dev < kMaxDevices) {
        int cur = done[dev].load(std::memory_order_relaxed);
        while (cur < bytes && !done[dev].compare_exchange_weak(cur, bytes, std::memory_order_release)) {
        }
    }
    return e;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16_bits(lo)) | (static_cast<uint32_t>(f32_to_bf16_bits(hi)) << 16);
}

// The 16-byte unit every kernel moves: one global or LDS vector access.
struct alignas(16) vec16 {
    uint32_t w[4];
};

__device__ __forceinline__ vec16 ld16(const void* p) {
    return *reinterpret_cast<const vec16*>(p);
}
__device__ __forceinline__ void st16(void* p, const vec16& v) {
    *reinterpret_cast<vec16*>(p) = v;
}

// Exclusive prefix sum of v[0..n) in LDS by one workgroup of NT threads
// (each thread sums a contiguous run, Hillis-Steele over the run totals).
// s_part: NT ints of LDS scratch. Ends with a barrier.
template <int NT>
__device__ void block_exclusive_scan(int* v, int n, int* s_part) {
    const int per = (n + NT - 1) / NT;
    const int b = threadIdx.x * per;
    int sum = 0;
    for (int i = 0; i < per; ++i)
        if (b + i < n) sum += v[b + i];
    s_part[threadIdx.x] = sum;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
        const int add = threadIdx.x >= off ? s_part[threadIdx.x - off] : 0;
        __syncthreads();
        s_part[threadIdx.x] += add;
        __syncthreads();
    }
    int run = s_part[threadIdx.x] - sum;
    for (int i = 0; i < per; ++i) {
        if (b + i < n) {
            const int c = v[b + i];
            v[b + i] = run;
            run += c;
        }
    }
    __syncthreads();
}

}  // namespace moe
