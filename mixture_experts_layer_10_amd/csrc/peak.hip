// Measurement helpers, not part of the layer: the matrix-core rate this chip
// actually sustains (and the shader clock it sustains it at), and the rate at
// which it streams a buffer in from HBM.
//
// Every compute unit gets two workgroups of four wavefronts (two wavefronts
// per SIMD). Each wavefront issues four independent chains of
// v_mfma_f32_32x32x16_bf16 (32768 FLOPs each), so the MFMA pipe of every SIMD
// always has an instruction whose operands are ready. The operands are
// pseudo-random bf16 values with random signs, because the power drawn, and
// so the clock the chip settles at, depends on the data's bit activity.
// Wavefront 0 of workgroup 0 reads the shader-clock counter and the constant
// 100 MHz real-time counter at its start and end; the ratio of the two spans
// is the shader clock over the loop.
#include <cstdint>

#include "moe_device.h"

namespace moe {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLoopThreads = 256;

// A bf16 of magnitude in [1, 2) with 7 random mantissa bits and a random sign.
__device__ __forceinline__ __bf16 rand_bf16(uint32_t h) {
    h ^= h >> 16;
    h *= 0x7feb352dU;
    h ^= h >> 15;
    h *= 0x846ca68bU;
    h ^= h >> 16;
    const uint16_t bits = static_cast<uint16_t>(((h & 1u) << 15) | (0x7fu << 7) | ((h >> 1) & 0x7fu));
    return __builtin_bit_cast(__bf16, bits);
}

__global__ __launch_bounds__(kLoopThreads, 2) void mfma_loop_kernel(int64_t iters, unsigned long long* out) {
    const uint32_t seed = (blockIdx.x * kLoopThreads + threadIdx.x) * 64u;
    bf16x8 a0, a1, b0, b1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a0[i] = rand_bf16(seed + i);
        a1[i] = rand_bf16(seed + 8 + i);
        b0[i] = rand_bf16(seed + 16 + i);
        b1[i] = rand_bf16(seed + 24 + i);
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const bool timer = blockIdx.x == 0 && threadIdx.x < 64;
    unsigned long long clk0 = 0, rt0 = 0;
    if (timer) {
        clk0 = __builtin_amdgcn_s_memtime();
        rt0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int64_t it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c3, 0, 0, 0);
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += c0[i] + c1[i] + c2[i] + c3[i];
    if (timer) {
        const unsigned long long clk1 = __builtin_amdgcn_s_memtime();
        const unsigned long long rt1 = __builtin_amdgcn_s_memrealtime();
        if (threadIdx.x == 0) {
            out[0] = clk1 - clk0;
            out[1] = rt1 - rt0;
            out[2] = static_cast<unsigned long long>(__builtin_bit_cast(uint32_t, sum));
        }
    }
}

// Reads every 16-byte granule of src once and folds them with XOR. Each
// workgroup takes blocks of kReadUnroll x 256 consecutive granules (sixteen
// independent 16-byte loads in flight per lane, so a block is 64 KB of
// consecutive memory), one workgroup per compute unit, blocks dealt round-
// robin; a tail shorter than a block is read granule by granule. Of the
// layouts, unroll depths and grid sizes tried on MI355X this streamed
// fastest. The fold is stored only where it matches a value a caller would
// not guess, so the loads cannot be dropped and almost nothing is written.
constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 16;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* src, int64_t n16, uint32_t* out) {
    constexpr int64_t kBlock = static_cast<int64_t>(kReadUnroll) * kReadThreads;
    const int64_t full = n16 / kBlock * kBlock;
    uint4 acc = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t b = static_cast<int64_t>(blockIdx.x) * kBlock; b < full; b += static_cast<int64_t>(gridDim.x) * kBlock) {
        uint4 v[kReadUnroll];
#pragma unroll
        for (int j = 0; j < kReadUnroll; ++j) v[j] = src[b + j * kReadThreads + threadIdx.x];
#pragma unroll
        for (int j = 0; j < kReadUnroll; ++j) {
            acc.x ^= v[j].x;
            acc.y ^= v[j].y;
            acc.z ^= v[j].z;
            acc.w ^= v[j].w;
        }
    }
    for (int64_t i = full + static_cast<int64_t>(blockIdx.x) * kReadThreads + threadIdx.x; i < n16;
         i += static_cast<int64_t>(gridDim.x) * kReadThreads) {
        const uint4 v = src[i];
        acc.x ^= v.x;
        acc.y ^= v.y;
        acc.z ^= v.z;
        acc.w ^= v.w;
    }
    const uint32_t f = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (f == 0x9e3779b9u) out[0] = f;
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* out, hipStream_t s) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t n16 = bytes / 16;
    const int64_t want = (n16 + kReadThreads - 1) / kReadThreads;
    const int64_t blocks = want < cus ? (want > 0 ? want : 1) : static_cast<int64_t>(cus);
    hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kReadThreads), 0, s,
                       static_cast<const uint4*>(src), n16, out);
    return hipGetLastError();
}

hipError_t launch_mfma_loop(int64_t iters, unsigned long long* out, double* flops, hipStream_t s) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t blocks = 2 * static_cast<int64_t>(cus);
    *flops = static_cast<double>(blocks) * (kLoopThreads / 64) * static_cast<double>(iters) * 4.0 * 32768.0;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kLoopThreads), 0, s, iters, out);
    return hipGetLastError();
}

}  // namespace moe
