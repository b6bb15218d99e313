// K3: dispatch. Builds per-expert counts and offsets and a stable
// permutation of the (token, slot) pairs into expert-contiguous order, for
// the local share of experts, with an optional per-expert capacity.
//
// What it computes: Perplexity "Lower latency and higher throughput with
// multi-node DeepSeek deployment", section "MoE Router" (dense dispatch and
// combine need the routing information aggregated per expert) and section
// "Expert parallelism" (each GPU owns 256/EP routed experts); Ultralytics
// glossary "Expert Parallelism", section "Load balancing and capacity" (an
// expert accepts at most a fixed multiple of its equal share; overflow
// tokens skip that expert). Order is (expert, token, slot); capacity is
// taken in token order.
//
// Three launches, no atomics whose order reaches a result:
//   1. per-chunk LDS histograms (a chunk is dispatch_chunk(P) consecutive pairs)
//      and per-chunk counts of expert ids outside [0, E);
//   2. one workgroup scans the histograms column-wise (per expert, over
//      chunks) and across experts -> raw counts, counts, offsets, and sums
//      the out-of-range counts into the workspace's error word;
//   3. per chunk, stable in-chunk ranks from wavefront ballots, then
//      row = offsets[e] + (earlier chunks' pairs of e) + in-chunk rank.
#include "moe_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
// Histograms up to this size are scanned from LDS. Kept small (with the
// 5 KB of static arrays, 17 KB) so that the one-workgroup scan fits on a CU
// beside a 256 x 256 GEMM workgroup of the shared expert (128-133 KB of the
// 160 KB), which may be running on a second stream; a larger request waits
// for such a workgroup to finish.
constexpr size_t kScanStageBytes = 12 * 1024;

__device__ __forceinline__ int local_expert(int id, int E, int begin, int El) {
    if (id < 0 || id >= E) return El;        // invalid id: treated as non-local
    const int le = id - begin;
    return (le >= 0 && le < El) ? le : El;   // El = "not local"
}

__global__ __launch_bounds__(kThreads) void hist_kernel(DispatchArgs a) {
    extern __shared__ int s_hist[];
    __shared__ int s_bad;
    const int El = a.El;
    for (int i = threadIdx.x; i < El; i += kThreads) s_hist[i] = 0;
    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    const int64_t cl = dispatch_chunk(a.P);
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * cl;
    const int64_t p1 = min(p0 + cl, a.P);
    int bad = 0;
    for (int64_t p = p0 + threadIdx.x; p < p1; p += kThreads) {
        const int id = a.ids[p];
        bad += (id < 0 || id >= a.E) ? 1 : 0;
        const int le = local_expert(id, a.E, a.begin, El);
        if (le < El) atomicAdd(&s_hist[le], 1);
    }
    if (bad) atomicAdd(&s_bad, bad);
    __syncthreads();
    int32_t* out = a.chunk_hist + static_cast<int64_t>(blockIdx.x) * El;
    for (int i = threadIdx.x; i < El; i += kThreads) out[i] = s_hist[i];
    if (threadIdx.x == 0) a.chunk_bad[blockIdx.x] = s_bad;     // written every call: nothing to clear
}

// Per expert, the running sum of its chunk histograms down the chunks (->
// chunk bases, raw count), then the capped counts and their exclusive scan
// across experts (-> offsets). With STAGED the histograms are first copied
// into LDS by coalesced loads, so the column walks read LDS instead of
// waiting on one global load per chunk.
template <bool STAGED>
__global__ __launch_bounds__(kThreads) void scan_kernel(DispatchArgs a, int nchunk) {
    __shared__ int s_off[4 * kThreads];
    __shared__ int s_part[kThreads];
    __shared__ int s_bad;
    extern __shared__ int s_hist[];                    // [nchunk * El] when STAGED
    const int El = a.El;
    const int64_t n = static_cast<int64_t>(nchunk) * El;
    // the batch's out-of-range ids: the chunks' counts summed here, the total
    // written after the barrier that follows the column walks
    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    {
        int bad = 0;
        for (int c = threadIdx.x; c < nchunk; c += kThreads) bad += a.chunk_bad[c];
        if (bad) atomicAdd(&s_bad, bad);
    }
    if constexpr (STAGED) {
        // sixteen independent loads in flight per thread, then their stores
        constexpr int kBatch = 16;
        for (int64_t b = threadIdx.x; b < n; b += kBatch * kThreads) {
            int v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int64_t i = b + j * kThreads;
                v[j] = i < n ? a.chunk_hist[i] : 0;
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int64_t i = b + j * kThreads;
                if (i < n) s_hist[i] = v[j];
            }
        }
        __syncthreads();
    }
    for (int e = threadIdx.x; e < El; e += kThreads) {
        // down the column in batches of eight chunks: the batch's reads are
        // independent, so only one read latency per batch is exposed
        int run = 0;
        for (int c0 = 0; c0 < nchunk; c0 += 8) {
            int h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t i = static_cast<int64_t>(c0 + j) * El + e;
                h[j] = c0 + j < nchunk ? (STAGED ? s_hist[i] : a.chunk_hist[i]) : 0;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (c0 + j < nchunk) {
                    a.chunk_base[static_cast<int64_t>(c0 + j) * El + e] = run;
                    run += h[j];
                }
            }
        }
        if (a.raw) a.raw[e] = run;
        const int cnt = static_cast<int64_t>(run) < a.cap ? run : static_cast<int>(a.cap);
        a.counts[e] = cnt;
        s_off[e] = cnt;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        s_part[0] = s_off[El - 1];                       // last count, kept for the total
        *a.bad_ids = s_bad;                              // written every call: nothing to clear
    }
    __syncthreads();
    const int last = s_part[0];
    __syncthreads();
    block_exclusive_scan<kThreads>(s_off, El, s_part);
    for (int e = threadIdx.x; e < El; e += kThreads) a.offsets[e] = s_off[e];
    if (threadIdx.x == 0) a.offsets[El] = s_off[El - 1] + last;
}

__global__ __launch_bounds__(kThreads) void scatter_kernel(DispatchArgs a) {
    extern __shared__ int s_mem[];
    const int El = a.El;
    int* s_run = s_mem;                    // [El]     pairs of e seen so far (whole batch)
    int* s_off = s_mem + El;               // [El]     offsets
    int* s_wcnt = s_mem + 2 * El;          // [4][El+1] per-wave counts of this step
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t chunk = blockIdx.x;
    for (int e = threadIdx.x; e < El; e += kThreads) {
        s_run[e] = a.chunk_base[chunk * El + e];
        s_off[e] = a.offsets[e];
    }
    for (int i = threadIdx.x; i < 4 * (El + 1); i += kThreads) s_wcnt[i] = 0;
    __syncthreads();

    int nbits = 1;
    while ((1 << nbits) <= El) ++nbits;    // enough bits for 0..El
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int64_t cl = dispatch_chunk(a.P);
    const int64_t p0 = chunk * cl;
    const int64_t p1 = min(p0 + cl, a.P);
    for (int64_t base = p0; base < p1; base += kThreads) {
        const int64_t p = base + threadIdx.x;
        const bool valid = p < p1;
        const int le = valid ? local_expert(a.ids[p], a.E, a.begin, El) : El;
        // lanes of this wave holding the same expert
        uint64_t same = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (le >> b) & 1;
            const uint64_t m = __ballot(bit);
            same &= bit ? m : ~m;
        }
        const int rank = __popcll(same & lt_mask);
        const int cnt = __popcll(same);
        if (valid && rank == cnt - 1) s_wcnt[wave * (El + 1) + le] = cnt;
        __syncthreads();
        if (valid) {
            int32_t row = -1;
            if (le < El) {
                int r = s_run[le] + rank;
                for (int w = 0; w < wave; ++w) r += s_wcnt[w * (El + 1) + le];
                if (static_cast<int64_t>(r) < a.cap) {
                    row = s_off[le] + r;
                    a.perm[row] = static_cast<int32_t>(p);
                }
            }
            a.inv[p] = row;
        }
        __syncthreads();
        for (int e = threadIdx.x; e < El; e += kThreads) {
            int add = 0;
            for (int w = 0; w < 4; ++w) {
                add += s_wcnt[w * (El + 1) + e];
                s_wcnt[w * (El + 1) + e] = 0;
            }
            s_run[e] += add;
        }
        if (threadIdx.x < 4) s_wcnt[threadIdx.x * (El + 1) + El] = 0;
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
    const int64_t nchunk = dispatch_chunks(a.P);
    if (nchunk == 0) return hipSuccess;
    hipLaunchKernelGGL(hist_kernel, dim3(static_cast<unsigned>(nchunk)), dim3(kThreads),
                       sizeof(int) * a.El, s, a);
    const size_t hist_bytes = sizeof(int) * static_cast<size_t>(nchunk) * a.El;
    if (hist_bytes <= kScanStageBytes)
        hipLaunchKernelGGL(scan_kernel<true>, dim3(1), dim3(kThreads), hist_bytes, s, a, static_cast<int>(nchunk));
    else
        hipLaunchKernelGGL(scan_kernel<false>, dim3(1), dim3(kThreads), 0, s, a, static_cast<int>(nchunk));
    const size_t lds = sizeof(int) * (2 * a.El + 4 * (a.El + 1));
    hipLaunchKernelGGL(scatter_kernel, dim3(static_cast<unsigned>(nchunk)), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace moe
