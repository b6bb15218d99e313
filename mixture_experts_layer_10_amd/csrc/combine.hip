// K7: combine. For every token, gathers its k expert output rows (through
// the inverse permutation), scales each by its gate, sums in fp32 and adds
// the shared expert's output.
//
// What it computes: Ultralytics glossary "Expert Parallelism", section "How
// tokens move between GPUs", step 4 (outputs return to the token's GPU and
// are summed weighted by the router scores); infra guide "Data parallelism
// and expert parallelism", section 3.1 step 4; the shared expert's output is
// added for every token (Perplexity "Lower latency and higher throughput
// with multi-node DeepSeek deployment", section "Expert parallelism").
// Dropped and non-local pairs (inv < 0) add nothing; gates are not
// renormalised.
//
// One workgroup per token; each thread moves 8 consecutive hidden elements
// per step with 16- or 32-byte accesses, so every row is read once,
// coalesced, and the token's rows are read concurrently (kBatch at a time).
#include "moe_device.h"

namespace moe {
namespace {

constexpr int kThreads = 128;
constexpr int kWideThreads = 448;      // rows of a multiple of 3584 columns
constexpr int kBatch = 8;             // pairs whose rows are in flight together

template <bool ROWS_F32>
__device__ __forceinline__ void load8(const void* base, int64_t off, float (&v)[8]) {
    if constexpr (ROWS_F32) {
        const vec16 a = ld16(static_cast<const float*>(base) + off);
        const vec16 b = ld16(static_cast<const float*>(base) + off + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = __uint_as_float(a.w[i]);
            v[4 + i] = __uint_as_float(b.w[i]);
        }
    } else {
        const vec16 a = ld16(static_cast<const uint16_t*>(base) + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_bits_to_f32(static_cast<uint16_t>(a.w[i] & 0xffffu));
            v[2 * i + 1] = bf16_bits_to_f32(static_cast<uint16_t>(a.w[i] >> 16));
        }
    }
}

// 8 row elements from their raw 16-byte pieces (two for fp32 rows, one for bf16).
template <bool ROWS_F32>
__device__ __forceinline__ void unpack8(const vec16 (&raw)[ROWS_F32 ? 2 : 1], float (&v)[8]) {
    if constexpr (ROWS_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = __uint_as_float(raw[0].w[i]);
            v[4 + i] = __uint_as_float(raw[ROWS_F32 ? 1 : 0].w[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_bits_to_f32(static_cast<uint16_t>(raw[0].w[i] & 0xffffu));
            v[2 * i + 1] = bf16_bits_to_f32(static_cast<uint16_t>(raw[0].w[i] >> 16));
        }
    }
}

template <bool ROWS_F32, bool OUT_F32, int NT>
__global__ __launch_bounds__(NT) void combine_kernel(CombineArgs a) {
    __shared__ int s_row[16];
    __shared__ float s_w[16];
    const int64_t t = blockIdx.x;
    const int k = a.k;
    if (threadIdx.x < k) {
        s_row[threadIdx.x] = a.inv[t * k + threadIdx.x];
        s_w[threadIdx.x] = a.w[t * k + threadIdx.x];
    }
    __syncthreads();
    const int H = a.H;
    for (int c = threadIdx.x * 8; c < H; c += NT * 8) {
        float acc[8];
        if (a.shared) {
            load8<true>(a.shared, t * H + c, acc);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        }
        // The rows of kBatch pairs are loaded, as raw 16-byte pieces, before
        // any is used, so their memory latencies overlap. A pair with no row
        // (inv < 0, or past k) loads row 0 (always allocated: T >= 1) and is
        // skipped when summing; the sum runs over j in order.
        constexpr int NV = ROWS_F32 ? 2 : 1;
        for (int j0 = 0; j0 < k; j0 += kBatch) {
            vec16 raw[kBatch][NV];
            int rr[kBatch];
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj) {
                rr[jj] = j0 + jj < k ? s_row[j0 + jj] : -1;
                const int64_t off = static_cast<int64_t>(rr[jj] < 0 ? 0 : rr[jj]) * H + c;
                if constexpr (ROWS_F32) {
                    raw[jj][0] = ld16(static_cast<const float*>(a.rows) + off);
                    raw[jj][NV - 1] = ld16(static_cast<const float*>(a.rows) + off + 4);
                } else {
                    raw[jj][0] = ld16(static_cast<const uint16_t*>(a.rows) + off);
                }
            }
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj) {
                if (rr[jj] >= 0) {
                    float v[8];
                    unpack8<ROWS_F32>(raw[jj], v);
                    const float wj = s_w[j0 + jj];
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] += wj * v[i];
                }
            }
        }
        if constexpr (OUT_F32) {
            float* y = static_cast<float*>(a.y) + t * H + c;
            st16(y, vec16{{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]), __float_as_uint(acc[3])}});
            st16(y + 4, vec16{{__float_as_uint(acc[4]), __float_as_uint(acc[5]), __float_as_uint(acc[6]), __float_as_uint(acc[7])}});
        } else {
            uint16_t* y = static_cast<uint16_t*>(a.y) + t * H + c;
            st16(y, vec16{{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                           pack_bf16x2(acc[6], acc[7])}});
        }
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(a.T));
    // A row of a multiple of 3584 columns (DeepSeek-V3's 7168) in two passes
    // of 448 threads: 0.510 against 0.527 ms for 128 threads (seven passes)
    // at the bf16 prefill layer.
    auto go = [&](auto nt_c) {
        constexpr int NT = decltype(nt_c)::value;
        const dim3 block(NT);
        if (a.rows_f32) {
            if (a.out_f32) hipLaunchKernelGGL((combine_kernel<true, true, NT>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((combine_kernel<true, false, NT>), grid, block, 0, s, a);
        } else {
            if (a.out_f32) hipLaunchKernelGGL((combine_kernel<false, true, NT>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((combine_kernel<false, false, NT>), grid, block, 0, s, a);
        }
    };
    if (a.H % (kWideThreads * 8) == 0) go(std::integral_constant<int, kWideThreads>{});
    else go(std::integral_constant<int, kThreads>{});
    return hipGetLastError();
}

}  // namespace moe
