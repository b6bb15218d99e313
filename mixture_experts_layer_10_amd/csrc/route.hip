// K2: scores, group-limited top-k and gates; one 64-lane wavefront per token.
//
// What it computes: NVIDIA "Optimizing DeepSeek R1 throughput on Blackwell",
// section "MoE layer optimisations > Top-K kernel fusion" (choose expert
// groups first, then the top 8 experts inside them, with a per-expert bias
// and a scaling factor); Ultralytics glossary "Expert Parallelism", section
// "Load balancing and capacity" (the bias only changes which experts are
// selected); Perplexity "Lower latency and higher throughput with multi-node
// DeepSeek deployment", section "MoE Router" (Mixtral routing = every group
// kept). The group score (sum of the two best experts), tie rules and the
// float32 exp recipe are this library's fixed reading; see moe.h.
//
// Every floating-point step that decides a selection is one IEEE float32
// operation: this file is built with -ffp-contract=off and the pragma below,
// and float division is HIP's default correctly rounded division.
#pragma clang fp contract(off)

#include <float.h>
#include <math.h>

#include "moe_device.h"

namespace moe {
namespace {

// Cody-Waite split of ln 2 (the high part has 15 significant bits, so
// n * kLn2Hi is exact for the |n| <= 126 used here) and 1/j! coefficients.
constexpr float kLn2Hi = 0.693145751953125f;
constexpr float kLn2Lo = static_cast<float>(0.6931471805599453094 - 0.693145751953125);
constexpr float kLog2e = static_cast<float>(1.0 / 0.6931471805599453094);
constexpr float kC8 = static_cast<float>(1.0 / 40320.0);
constexpr float kC7 = static_cast<float>(1.0 / 5040.0);
constexpr float kC6 = static_cast<float>(1.0 / 720.0);
constexpr float kC5 = static_cast<float>(1.0 / 120.0);
constexpr float kC4 = static_cast<float>(1.0 / 24.0);
constexpr float kC3 = static_cast<float>(1.0 / 6.0);
constexpr float kC2 = 0.5f;
constexpr float kC1 = 1.0f;
constexpr float kC0 = 1.0f;

// e**y for y <= 0: clamp to -87, n = rint(y log2 e), r = (y - n ln2_hi) -
// n ln2_lo, degree-8 Taylor polynomial of e**r in Horner form, ldexp.
__device__ __forceinline__ float exp_neg(float y) {
    y = y < -87.0f ? -87.0f : y;
    const float n = rintf(y * kLog2e);
    const float r = (y - n * kLn2Hi) - n * kLn2Lo;
    float p = kC8;
    p = p * r + kC7;
    p = p * r + kC6;
    p = p * r + kC5;
    p = p * r + kC4;
    p = p * r + kC3;
    p = p * r + kC2;
    p = p * r + kC1;
    p = p * r + kC0;
    return ldexpf(p, static_cast<int>(n));
}

__device__ __forceinline__ float sigmoid_fixed(float x) {
    if (x >= 0.0f) {
        const float e = exp_neg(-x);
        return 1.0f / (1.0f + e);
    }
    const float e = exp_neg(x);
    return e / (1.0f + e);
}

// (v, i) beats (w, j) when v > w, or v == w and i < j.
__device__ __forceinline__ bool better(float v, int i, float w, int j) {
    return v > w || (v == w && i < j);
}

// One step of the arg-max reduction: take the pair DPP control CTRL brings
// from another lane if it is better; lanes CTRL gives no source (or rows
// outside ROW_MASK) compare with their own pair and keep it.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_dpp(float& v, int& i) {
    const int vb = __builtin_bit_cast(int, v);
    const float ov = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(vb, vb, CTRL, ROW_MASK, 0xf, false));
    const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, ROW_MASK, 0xf, false);
    if (better(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}

// Arg-max over the 64 lanes with the gfx9 DPP reduction (row_shr 1, 2, 4, 8
// within each 16-lane row, then row_bcast 15 and 31 across rows) into lane
// 63, read back as a wave-uniform pair. "better" is a total order on (value,
// index), so the winner does not depend on the reduction order.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    argmax_dpp<0x111, 0xf>(v, i);        // row_shr:1
    argmax_dpp<0x112, 0xf>(v, i);        // row_shr:2
    argmax_dpp<0x114, 0xf>(v, i);        // row_shr:4
    argmax_dpp<0x118, 0xf>(v, i);        // row_shr:8  (lane 15 of each row: the row's best)
    argmax_dpp<0x142, 0xa>(v, i);        // row_bcast:15 into rows 1 and 3
    argmax_dpp<0x143, 0xc>(v, i);        // row_bcast:31 into rows 2 and 3 (lane 63: the best)
    v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
    i = __builtin_amdgcn_readlane(i, 63);
}

constexpr int kMaxE = 512;

// One workgroup = one wavefront = one token. Lane l owns experts
// l*EPL .. l*EPL+EPL-1.
template <int EPL>
__global__ __launch_bounds__(64) void route_kernel(RouteArgs a) {
    __shared__ float s_sel[kMaxE];      // selection score (score + bias)
    __shared__ float s_score[kMaxE];    // unbiased score (sigmoid) / logit
    __shared__ float s_logit[kMaxE];
    __shared__ int s_ids[16];
    const int lane = threadIdx.x;
    const int64_t t = blockIdx.x;
    const int E = a.E;
    const float* lrow = a.logits + t * E;

    float sel[EPL];
    int idx[EPL];
    // all of this lane's logits (and biases) are loaded before any is used,
    // so the loads are in flight together (indices past E read the last
    // expert again; those values are not used)
    float lv[EPL], bv[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) lv[q] = lrow[min(lane * EPL + q, E - 1)];
    if (a.score_bias) {
#pragma unroll
        for (int q = 0; q < EPL; ++q) bv[q] = a.score_bias[min(lane * EPL + q, E - 1)];
    }
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
        const int e = lane * EPL + q;
        if (e < E) {
            const float l = lv[q];
            const float sc = a.score_fn == MOE_SCORE_SIGMOID ? sigmoid_fixed(l) : l;
            const float v = a.score_bias ? sc + bv[q] : sc;
            s_logit[e] = l;
            s_score[e] = sc;
            s_sel[e] = v;
            sel[q] = v;
            idx[q] = e;
        } else {
            sel[q] = -INFINITY;
            idx[q] = 0x7fffffff;
        }
    }
    __syncthreads();

    // Group limit: lane g < G scans its group for the two best selection
    // scores; G_k rounds of arg-max keep the best groups.
    if (a.Gk < a.G) {
        const int gs = E / a.G;
        float gscore = -INFINITY;
        int gid = 0x7fffffff;
        const int lpg = gs / EPL;                       // lanes per group, when whole
        if (gs % EPL == 0 && lpg >= 1 && lpg <= 64 && (lpg & (lpg - 1)) == 0 && E == 64 * EPL) {
            // each lane's two best, then a butterfly over the group's lanes:
            // the top two of a union of two top-twos (t1 >= t2, o1 >= o2) are
            // max(t1, o1) and max(min(t1, o1), max(t2, o2))
            float t1 = -INFINITY, t2 = -INFINITY;
#pragma unroll
            for (int q = 0; q < EPL; ++q) {
                const float v = s_sel[lane * EPL + q];
                if (v > t1) {
                    t2 = t1;
                    t1 = v;
                } else if (v > t2) {
                    t2 = v;
                }
            }
            for (int off = 1; off < lpg; off <<= 1) {
                const float o1 = __shfl_xor(t1, off, 64);
                const float o2 = __shfl_xor(t2, off, 64);
                const float n1 = fmaxf(t1, o1);
                t2 = fmaxf(fminf(t1, o1), fmaxf(t2, o2));
                t1 = n1;
            }
            if (lane % lpg == 0) {
                gscore = gs >= 2 ? t1 + t2 : t1;
                gid = lane / lpg;
            }
        } else if (lane < a.G) {
            float t1 = -INFINITY, t2 = -INFINITY;
            for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
                const float v = s_sel[e];
                if (v > t1) {
                    t2 = t1;
                    t1 = v;
                } else if (v > t2) {
                    t2 = v;
                }
            }
            gscore = gs >= 2 ? t1 + t2 : t1;
            gid = lane;
        }
        uint64_t keep = 0;
        for (int r = 0; r < a.Gk; ++r) {
            float v = gscore;
            int i = gid;
            wave_argmax(v, i);
            keep |= 1ull << i;
            if (gid == i) {                             // the lane that holds group i
                gscore = -INFINITY;
                gid = 0x7fffffff;
            }
        }
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
            if (idx[q] < E && !((keep >> (idx[q] / gs)) & 1ull)) {
                sel[q] = -INFINITY;
                idx[q] = 0x7fffffff;
            }
        }
    }

    // k rounds of arg-max over the allowed experts.
    for (int r = 0; r < a.k; ++r) {
        float v = -INFINITY;
        int i = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
            if (better(sel[q], idx[q], v, i)) {
                v = sel[q];
                i = idx[q];
            }
        }
        wave_argmax(v, i);
        if (lane == 0) s_ids[r] = i;
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
            if (idx[q] == i) {
                sel[q] = -INFINITY;
                idx[q] = 0x7fffffff;
            }
        }
    }
    __syncthreads();

    // Gates, in slot order, by lane 0 (sequential sums fix the rounding).
    if (lane == 0) {
        const int k = a.k;
        float g[16];
        if (a.score_fn == MOE_SCORE_SIGMOID) {
            float tot = 0.0f;
            for (int j = 0; j < k; ++j) {
                g[j] = s_score[s_ids[j]];
                tot = tot + g[j];
            }
            if (a.renorm)
                for (int j = 0; j < k; ++j) g[j] = g[j] / tot;
        } else {
            float m, tot = 0.0f;
            if (a.renorm) {
                m = s_logit[s_ids[0]];
                for (int j = 1; j < k; ++j) m = fmaxf(m, s_logit[s_ids[j]]);
                for (int j = 0; j < k; ++j) {
                    g[j] = exp_neg(s_logit[s_ids[j]] - m);
                    tot = tot + g[j];
                }
            } else {
                m = s_logit[0];
                for (int e = 1; e < E; ++e) m = fmaxf(m, s_logit[e]);
                for (int e = 0; e < E; ++e) tot = tot + exp_neg(s_logit[e] - m);
                for (int j = 0; j < k; ++j) g[j] = exp_neg(s_logit[s_ids[j]] - m);
            }
            for (int j = 0; j < k; ++j) g[j] = g[j] / tot;
        }
        for (int j = 0; j < k; ++j) {
            if (a.gamma != 1.0f) g[j] = g[j] * a.gamma;
            a.ids[t * k + j] = s_ids[j];
            a.w[t * k + j] = g[j];
        }
    }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(a.T)), block(64);
    if (a.E <= 64)
        hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, a);
    else if (a.E <= 128)
        hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, a);
    else if (a.E <= 256)
        hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
