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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// float -> bf16 bits, rounded to nearest even: one v_cvt_pk_bf16_f32 on
// gfx950 (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats -> packed bf16 (lo in the low half), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// SwiGLU's activation product silu(g) * u = g * u / (1 + e^-g), with the
// hardware exponential and reciprocal (1 ulp each) instead of a correctly
// rounded division: six instructions, two of them transcendental, where the
// division alone took ten. Every SwiGLU epilogue uses this one definition.
// For g -> -inf the reciprocal of +inf gives 0, so the product is +-0.
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
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

// Buffer descriptor of a raw byte range (word 3: data format 32, the one a
// raw buffer access needs on this generation): loads through it take the
// base from scalar registers and a 32-bit offset per lane.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_buffer(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                             0x00020000);
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ vec16 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
    return __builtin_bit_cast(vec16, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// 16 bytes per lane from a buffer straight into LDS (wave base lds_wave_base)
__device__ __forceinline__ void buf_load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff,
                                               unsigned char* lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff, soff,
                                             0, 0);
}

// Exclusive prefix sum of v[0..n) in LDS by one workgroup of NT threads
// (each thread sums a contiguous run, Hillis-Steele over the run totals).
// s_part: NT values of LDS scratch. Ends with a barrier.
template <int NT, typename V>
__device__ void block_exclusive_scan(V* v, int n, V* s_part) {
    const int per = (n + NT - 1) / NT;
    const int b = threadIdx.x * per;
    V sum = 0;
    for (int i = 0; i < per; ++i)
        if (b + i < n) sum += v[b + i];
    s_part[threadIdx.x] = sum;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
        const V add = threadIdx.x >= off ? s_part[threadIdx.x - off] : V{0};
        __syncthreads();
        s_part[threadIdx.x] += add;
        __syncthreads();
    }
    V run = s_part[threadIdx.x] - sum;
    for (int i = 0; i < per; ++i) {
        if (b + i < n) {
            const V c = v[b + i];
            v[b + i] = run;
            run += c;
        }
    }
    __syncthreads();
}

}  // namespace moe
