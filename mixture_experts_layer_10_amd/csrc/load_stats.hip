// Expert load statistics (device) and the redundant-expert placement planner
// (host), after the infra guide "Data parallelism and expert parallelism",
// section 5: under expert parallelism a layer waits for the GPU with the most
// tokens, so the load each expert receives is recorded every step and, from
// time to time, experts are re-placed and the hottest ones replicated
// (section 5.3), with the greedy rule of section 5.2.
//
//  * expert_load_kernel: histogram of the router's top-k ids over all E
//    experts (the router sees every expert, whatever share a GPU holds),
//    accumulated into an int64 per expert; integer atomics, so the result
//    is exact and order-independent.
//  * plan_placement: extra replicas one at a time to the expert with the
//    largest load per replica; replicas heaviest first onto the least-loaded
//    GPU that still has a free slot. Ties go to the lowest expert id and the
//    lowest GPU index; equal replica loads keep (expert, replica) order.
#include <algorithm>
#include <cstdint>
#include <numeric>
#include <vector>

#include "moe_device.h"

namespace moe {
namespace {

constexpr int kLoadThreads = 256;

__global__ __launch_bounds__(kLoadThreads) void expert_load_kernel(const int32_t* ids, int64_t n, int E,
                                                                   unsigned long long* load) {
    extern __shared__ unsigned int s_hist[];           // E counters
    for (int e = threadIdx.x; e < E; e += kLoadThreads) s_hist[e] = 0u;
    __syncthreads();
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kLoadThreads + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kLoadThreads) {
        const int e = ids[i];
        if (e >= 0 && e < E) atomicAdd(&s_hist[e], 1u);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kLoadThreads)
        if (s_hist[e]) atomicAdd(&load[e], static_cast<unsigned long long>(s_hist[e]));
}

}  // namespace

hipError_t launch_expert_load(const int32_t* ids, int64_t n, int E, int64_t* load, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + kLoadThreads * 16 - 1) / (kLoadThreads * 16), 1024);
    hipLaunchKernelGGL(expert_load_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kLoadThreads),
                       static_cast<size_t>(E) * sizeof(unsigned int), s, ids, n, E,
                       reinterpret_cast<unsigned long long*>(load));
    return hipGetLastError();
}

void plan_placement(const int64_t* load, int E, int ranks, int redundant, int32_t* replicas, int32_t* slot_expert,
                    double* rank_load) {
    for (int e = 0; e < E; ++e) replicas[e] = 1;
    // extra replicas: largest load per replica, compared exactly as
    // load[a] * replicas[b] > load[b] * replicas[a]
    for (int r = 0; r < redundant; ++r) {
        int best = 0;
        for (int e = 1; e < E; ++e)
            if (static_cast<__int128>(load[e]) * replicas[best] > static_cast<__int128>(load[best]) * replicas[e])
                best = e;
        ++replicas[best];
    }
    // replicas in creation order (expert, then replica), then heaviest first
    struct Piece {
        double w;
        int e;
    };
    std::vector<Piece> pieces;
    pieces.reserve(static_cast<size_t>(E) + redundant);
    for (int e = 0; e < E; ++e) {
        const double w = static_cast<double>(load[e]) / static_cast<double>(replicas[e]);
        for (int k = 0; k < replicas[e]; ++k) pieces.push_back({w, e});
    }
    std::stable_sort(pieces.begin(), pieces.end(), [](const Piece& a, const Piece& b) { return a.w > b.w; });
    const int per_rank = (E + redundant) / ranks;
    std::vector<int> used(ranks, 0);
    for (int g = 0; g < ranks; ++g) rank_load[g] = 0.0;
    for (const Piece& p : pieces) {
        int pick = -1;
        for (int g = 0; g < ranks; ++g)
            if (used[g] < per_rank && (pick < 0 || rank_load[g] < rank_load[pick])) pick = g;
        rank_load[pick] += p.w;
        slot_expert[pick * per_rank + used[pick]] = p.e;
        ++used[pick];
    }
}

}  // namespace moe
