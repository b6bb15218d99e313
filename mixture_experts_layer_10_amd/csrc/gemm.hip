// K1 / K5 / K6: grouped GEMM on gfx950 MFMA.
//
// What it computes (Perplexity "Lower latency and higher throughput with
// multi-node DeepSeek deployment", section "Roofline > GroupGEMM"): g groups,
// group i multiplies its [m_i, k] rows by a [k, n] weight. Here a group is a
// local routed expert (its rows are the dispatched (token, slot) pairs) or
// the shared expert (every token). Two epilogues:
//   SWIGLU  C[r, n] = silu(A_r . Wgate[n]) * (A_r . Wup[n])   (gate/up GEMM,
//           infra guide "Data parallelism and expert parallelism", section
//           2.1: an expert is gate, up and down matrices; SiLU per the
//           Perplexity section "Quantization");
//   PLAIN   C[r, n] = A_r . W[n] (+ bias[n])                  (down GEMM, and
//           the router GEMM with bf16 in and fp32 out, NVIDIA "Optimizing
//           DeepSeek R1 throughput on Blackwell", "mixed I/O RouterGEMM").
// Group sizes come from device memory (the dispatch offsets), so the launch
// needs no host synchronisation (Perplexity, section "Quantization": kernels
// driven by per-expert token counts rather than buffer sizes).
//
// Design (MI355X, CDNA4):
//  * a workgroup = 4 wavefronts computes a BM x 256-column tile (SWIGLU: 128
//    gate + 128 up columns -> 128 h columns); each wavefront owns 64 weight
//    columns and all BM rows;
//  * weights (the streamed operand) go straight from HBM into VGPRs in MFMA
//    operand order, PD chunks ahead of use (register ring, no LDS);
//  * the activation tile (gathered through the dispatch permutation) is
//    staged once per chunk into double-buffered LDS with an XOR swizzle and
//    shared by the 4 wavefronts;
//  * v_mfma_f32_16x16x32_bf16 (bf16) / v_mfma_f32_16x16x4_f32 (fp32); 16-row
//    blocks beyond a tile's real row count are skipped;
//  * tiles are remapped so consecutive tiles of one expert land on one XCD
//    (the hardware deals workgroups round-robin over the 8 XCDs), so that an
//    expert's activation rows are read from HBM once per XCD L2.
//
// K-ordering: each lane's A and B registers hold the same K positions, so
// the MFMA's internal K order does not matter: in every chunk, lane group
// q = lane/16 holds a contiguous run of K positions; MFMA s of the chunk uses
// the s-th sub-run of every lane group, identically for A and B.
#include <float.h>

#include <algorithm>

#include "moe_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <Elem EL>
struct Tr;
template <>
struct Tr<Elem::BF16> {
    static constexpr int kElemBytes = 2;
    static constexpr int kRunG = 4;        // 16-byte granules per lane run
    static constexpr int kRowG = 16;       // granules per LDS row (one chunk)
    static constexpr int kChunk = kRowG * 16 / kElemBytes;   // 128 K positions
};
template <>
struct Tr<Elem::F32> {
    static constexpr int kElemBytes = 4;
    static constexpr int kRunG = 4;
    static constexpr int kRowG = 16;
    static constexpr int kChunk = kRowG * 16 / kElemBytes;   // 64 K positions
};

__device__ __forceinline__ bf16x8 as_bf16x8(const vec16& v) {
    return __builtin_bit_cast(bf16x8, v);
}

template <Elem EL>
__device__ __forceinline__ void mfma_granule(const vec16& a, const vec16& b, f32x4& acc);

template <>
__device__ __forceinline__ void mfma_granule<Elem::BF16>(const vec16& a, const vec16& b, f32x4& acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), acc, 0, 0, 0);
}
template <>
__device__ __forceinline__ void mfma_granule<Elem::F32>(const vec16& a, const vec16& b, f32x4& acc) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w[c]), __uint_as_float(b.w[c]), acc, 0, 0, 0);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + __expf(-g)) * u;
}

template <Elem EL, Epi EPI, int BM, int PD>
__global__ __launch_bounds__(kThreads, (BM <= 64 ? 2 : 1)) void gemm_kernel(GemmArgs a, int n_tiles) {
    using T = Tr<EL>;
    constexpr int EB = T::kElemBytes;
    constexpr int RUNG = T::kRunG;
    constexpr int ROWG = T::kRowG;
    constexpr int ROWB = ROWG * 16;                    // LDS bytes per tile row
    constexpr int NRF = BM / 16;                       // 16-row blocks
    constexpr int ROWS_PER_PASS = kThreads / ROWG;     // A rows loaded per pass
    constexpr int PASSES = BM / ROWS_PER_PASS;
    constexpr int NB = PD + 1;                         // B register buffers
    constexpr int U = (NB % 2 == 0) ? NB : 2 * NB;     // unroll: both ring indices static
    static_assert(BM % ROWS_PER_PASS == 0, "tile rows");

    __shared__ __attribute__((aligned(16))) unsigned char s_a[2][BM * ROWB];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;

    // ---- tile lookup -----------------------------------------------------
    // Work items are (group, n-tile, m-tile, k-slice), k-slice fastest, then
    // m-tile: the blocks that stream the same weight panel run side by side.
    // Items are dealt to the 8 XCDs in contiguous ranges (the hardware deals
    // blocks round-robin), so neighbouring items share an XCD's L2.
    const int KS = a.ksplit;
    const int n_groups = a.n_local + a.has_shared;
    const int per_item = n_tiles * KS;                 // items per m-tile
    // A null schedule means a single group of T rows.
    const int total = (a.sched ? a.sched[n_groups] : (a.T + BM - 1) / BM) * per_item;
    const int per_xcd = (total + 7) >> 3;
    const int slot = static_cast<int>(blockIdx.x >> 3);
    if (slot >= per_xcd) return;
    const int L = static_cast<int>(blockIdx.x & 7) * per_xcd + slot;
    if (L >= total) return;
    int g = 0, mt_begin = 0, mt_count = (a.T + BM - 1) / BM;
    if (a.sched) {
        int lo = 0, hi = n_groups;                     // sched[lo]*per_item <= L < sched[hi]*per_item
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.sched[mid] * per_item <= L) lo = mid; else hi = mid;
        }
        g = lo;
        mt_begin = a.sched[g];
        mt_count = a.sched[g + 1] - mt_begin;
    }
    const int local = L - mt_begin * per_item;
    const int ks = local % KS;
    const int nt = (local / KS) / mt_count;
    const int mt = (local / KS) - nt * mt_count;
    const bool shared = a.has_shared && g == a.n_local;
    int row0 = 0, rows_g = a.T;
    if (!shared && a.offsets) {
        row0 = a.offsets[g];
        rows_g = a.offsets[g + 1] - row0;
    }
    const int m0 = mt * BM;
    const int rows = min(BM, rows_g - m0);
    const int nrf = (rows + 15) >> 4;
    const int K = a.K;
    const int nch_all = K / T::kChunk;
    const int c_begin = (nch_all * ks) / KS;
    const int nch = (nch_all * (ks + 1)) / KS - c_begin;

    // ---- B (weights): per-lane pointers of the 4 column fragments ----------
    const unsigned char* Bg = shared ? static_cast<const unsigned char*>(a.B_shared)
                                     : static_cast<const unsigned char*>(a.B) + static_cast<int64_t>(g) * a.b_stride * EB;
    const unsigned char* bptr[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        int brow;
        if constexpr (EPI == Epi::SWIGLU) {
            const int n0 = nt * 128 + wave * 32;
            brow = (f < 2) ? n0 + 16 * f + lr : a.inter + n0 + 16 * (f - 2) + lr;
        } else {
            brow = nt * 256 + wave * 64 + 16 * f + lr;
            brow = brow < a.N ? brow : a.N - 1;        // column tail: valid row, result dropped
        }
        bptr[f] = Bg + (static_cast<int64_t>(brow) * K) * EB + lq * RUNG * 16 + static_cast<int64_t>(c_begin) * ROWB;
    }

    // ---- A (activations): per-thread row sources for the LDS fill ----------
    const unsigned char* Abase = static_cast<const unsigned char*>(shared ? a.A_shared : a.A);
    const int aj = tid % ROWG;                         // granule within the row
    const int ar = tid / ROWG;                         // first row of this thread
    const unsigned char* asrc[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        int r = ar + i * ROWS_PER_PASS;
        r = r < rows ? r : rows - 1;                   // rows past the end: a valid row, unused
        int64_t src_row;
        if (shared) src_row = m0 + r;
        else if (a.gather) src_row = a.perm[row0 + m0 + r] / a.topk;
        else src_row = row0 + m0 + r;
        asrc[i] = Abase + (src_row * K) * EB + aj * 16 + static_cast<int64_t>(c_begin) * ROWB;
    }
    // LDS store offset (row ar, swizzled granule); pass i adds i*ROWS_PER_PASS rows.
    const int a_st = ar * ROWB + ((aj ^ (ar & (ROWG - 1))) * 16);
    // LDS read offsets for sub-run s of this lane (row lr of each 16-row block).
    int a_ld[RUNG];
#pragma unroll
    for (int s = 0; s < RUNG; ++s) a_ld[s] = lr * ROWB + (((lq * RUNG + s) ^ lr) * 16);

    f32x4 acc[NRF][4];
#pragma unroll
    for (int i = 0; i < NRF; ++i)
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    vec16 breg[NB][4][RUNG];
    vec16 areg[2][PASSES];

    auto load_b = [&](vec16 (&dst)[4][RUNG], int c) {
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int s = 0; s < RUNG; ++s) dst[f][s] = ld16(bptr[f] + static_cast<int64_t>(c) * ROWB + s * 16);
    };
    auto load_a = [&](vec16 (&dst)[PASSES], int c) {
#pragma unroll
        for (int i = 0; i < PASSES; ++i) dst[i] = ld16(asrc[i] + static_cast<int64_t>(c) * ROWB);
    };
    auto store_a = [&](const vec16 (&src)[PASSES], int buf) {
#pragma unroll
        for (int i = 0; i < PASSES; ++i) st16(&s_a[buf][a_st + i * ROWS_PER_PASS * ROWB], src[i]);
    };
    auto compute = [&](const vec16 (&b)[4][RUNG], int buf) {
#pragma unroll
        for (int i = 0; i < NRF; ++i) {
            if (i < nrf) {
#pragma unroll
                for (int s = 0; s < RUNG; ++s) {
                    const vec16 av = ld16(&s_a[buf][i * 16 * ROWB + a_ld[s]]);
#pragma unroll
                    for (int f = 0; f < 4; ++f) mfma_granule<EL>(av, b[f][s], acc[i][f]);
                }
            }
        }
    };

    // ---- main loop ---------------------------------------------------------
    // Chunk c's activations: global -> VGPR two iterations ahead, VGPR -> LDS
    // at the end of iteration c-1. Chunk c's weights: global -> VGPR PD
    // iterations ahead. Loads are issued oldest-needed first, so each wait
    // leaves the younger loads in flight.
    if (nch > 0) {
        load_a(areg[0], 0);
        if (nch > 1) load_a(areg[1], 1);
#pragma unroll
        for (int p = 0; p < PD; ++p)
            if (p < nch) load_b(breg[p], p);
        store_a(areg[0], 0);
        __syncthreads();
    }
    for (int c0 = 0; c0 < nch; c0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u;
            if (c < nch) {
                if (c + 2 < nch) load_a(areg[u & 1], c + 2);
                if (c + PD < nch) load_b(breg[(u + PD) % NB], c + PD);
                compute(breg[u % NB], u & 1);
                if (c + 1 < nch) store_a(areg[(u + 1) & 1], (u + 1) & 1);
                __syncthreads();
            }
        }
    }

    // ---- epilogue ------------------------------------------------------------
    const int64_t crow0 = shared ? m0 : static_cast<int64_t>(row0) + m0;
    unsigned char* Cb = static_cast<unsigned char*>(shared ? a.C_shared : a.C);
    if constexpr (EPI == Epi::SWIGLU) {
#pragma unroll
        for (int i = 0; i < NRF; ++i) {
            if (i < nrf) {
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    const int col = nt * 128 + wave * 32 + 16 * f + lr;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int r = i * 16 + lq * 4 + v;
                        if (r < rows) {
                            const float h = silu_mul(acc[i][f][v], acc[i][f + 2][v]);
                            const int64_t off = (crow0 + r) * a.ldc + col;
                            if constexpr (EL == Elem::F32)
                                reinterpret_cast<float*>(Cb)[off] = h;
                            else
                                reinterpret_cast<uint16_t*>(Cb)[off] = f32_to_bf16_bits(h);
                        }
                    }
                }
            }
        }
    } else {
        const bool split = KS > 1;
        float* P = split ? a.partial + static_cast<int64_t>(ks) * a.T * a.ldc : nullptr;
#pragma unroll
        for (int i = 0; i < NRF; ++i) {
            if (i < nrf) {
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const int col = nt * 256 + wave * 64 + 16 * f + lr;
                    if (col < a.N) {
                        const float bias = (!split && a.bias) ? a.bias[col] : 0.0f;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int r = i * 16 + lq * 4 + v;
                            if (r < rows) {
                                const float o = acc[i][f][v] + bias;
                                const int64_t off = (crow0 + r) * a.ldc + col;
                                if (split)
                                    P[off] = o;
                                else if (a.out_f32)
                                    reinterpret_cast<float*>(Cb)[off] = o;
                                else
                                    reinterpret_cast<uint16_t*>(Cb)[off] = f32_to_bf16_bits(o);
                            }
                        }
                    }
                }
            }
        }
    }
}

// C[t][n] = bias[n] + sum over K slices of partial[s][t][n] (fp32).
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(GemmArgs a) {
    const int64_t n = static_cast<int64_t>(a.T) * a.ldc;
    const int64_t stride = n;
    for (int64_t i = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * 4; i < n;
         i += static_cast<int64_t>(gridDim.x) * kThreads * 4) {
        vec16 acc = ld16(a.partial + i);
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = __uint_as_float(acc.w[j]);
        for (int s = 1; s < a.ksplit; ++s) {
            const vec16 p = ld16(a.partial + s * stride + i);
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] += __uint_as_float(p.w[j]);
        }
        if (a.bias) {
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] += a.bias[(i + j) % a.ldc];
        }
        st16(static_cast<float*>(a.C) + i,
             vec16{{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])}});
    }
}

// m-tile prefix over the groups: sched[g] = sum_{g' < g} ceil(rows_g' / bm).
__global__ __launch_bounds__(kThreads) void schedule_kernel(GemmArgs a, int bm, int32_t* sched) {
    __shared__ int s_v[4 * kThreads + 4];
    __shared__ int s_part[kThreads];
    const int n_groups = a.n_local + a.has_shared;
    for (int g = threadIdx.x; g < n_groups; g += kThreads) {
        int rows = a.T;
        if (!(a.has_shared && g == a.n_local) && a.offsets) rows = a.offsets[g + 1] - a.offsets[g];
        s_v[g] = (rows + bm - 1) / bm;
    }
    __syncthreads();
    if (threadIdx.x == 0) s_part[0] = s_v[n_groups - 1];
    __syncthreads();
    const int last = s_part[0];
    __syncthreads();
    block_exclusive_scan<kThreads>(s_v, n_groups, s_part);
    for (int g = threadIdx.x; g < n_groups; g += kThreads) sched[g] = s_v[g];
    if (threadIdx.x == 0) sched[n_groups] = s_v[n_groups - 1] + last;
}

template <Elem EL, Epi EPI, int BM, int PD>
void launch_one(const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    hipLaunchKernelGGL((gemm_kernel<EL, EPI, BM, PD>), dim3(static_cast<unsigned>(p.grid)), dim3(kThreads), 0, s,
                       a, p.n_tiles);
}

template <Elem EL, Epi EPI>
hipError_t launch_bm(GemmArgs a, const GemmPlan& p, hipStream_t s) {
    a.ksplit = p.ksplit < 1 ? 1 : p.ksplit;
    switch (p.bm) {
        case 32: launch_one<EL, EPI, 32, 1>(a, p, s); break;
        case 64: launch_one<EL, EPI, 64, 1>(a, p, s); break;
        case 128: launch_one<EL, EPI, 128, 1>(a, p, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

GemmPlan plan_gemm(Elem e, Epi epi, int64_t rows_upper, int n_groups, int64_t expected_rows_per_group, int N) {
    (void)e;
    GemmPlan p;
    p.bm = expected_rows_per_group <= 32 ? 32 : expected_rows_per_group <= 64 ? 64 : 128;
    const int cols_per_tile = epi == Epi::SWIGLU ? 128 : 256;
    p.n_tiles = (N + cols_per_tile - 1) / cols_per_tile;
    p.ksplit = 1;
    // sum_g ceil(rows_g / bm) <= rows_upper / bm + n_groups
    const int64_t m_tiles = rows_upper / p.bm + n_groups;
    p.grid = ((m_tiles * p.n_tiles + 7) / 8) * 8;
    return p;
}

GemmPlan plan_dense_splitk(int64_t T, int N, int K, int chunk) {
    GemmPlan p;
    p.bm = T <= 32 ? 32 : T <= 1024 ? 64 : 128;
    p.n_tiles = (N + 255) / 256;
    const int64_t tiles = (T + p.bm - 1) / p.bm * p.n_tiles;
    const int nch = K / chunk;
    // aim for >= 512 workgroups, each slice at least 4 chunks long
    int ks = 1;
    while (N % 4 == 0 && ks < 16 && tiles * ks < 512 && nch / (ks * 2) >= 4) ks *= 2;
    p.ksplit = ks;
    p.grid = ((tiles * ks + 7) / 8) * 8;
    return p;
}

hipError_t launch_splitk_reduce(const GemmArgs& a, int ksplit, hipStream_t s) {
    if (ksplit <= 1) return hipSuccess;
    const int64_t n4 = (static_cast<int64_t>(a.T) * a.ldc + 3) / 4;
    const int64_t blocks = std::min<int64_t>((n4 + kThreads - 1) / kThreads, 4096);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_schedule(const GemmArgs& a, int bm, int32_t* sched, hipStream_t s) {
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kThreads), 0, s, a, bm, sched);
    return hipGetLastError();
}

hipError_t launch_gemm(Elem e, Epi epi, const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    if (p.grid == 0) return hipSuccess;
    if (e == Elem::BF16)
        return epi == Epi::SWIGLU ? launch_bm<Elem::BF16, Epi::SWIGLU>(a, p, s) : launch_bm<Elem::BF16, Epi::PLAIN>(a, p, s);
    if (e == Elem::F32)
        return epi == Epi::SWIGLU ? launch_bm<Elem::F32, Epi::SWIGLU>(a, p, s) : launch_bm<Elem::F32, Epi::PLAIN>(a, p, s);
    return hipErrorInvalidValue;
}

}  // namespace moe
