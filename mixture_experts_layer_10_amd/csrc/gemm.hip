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
// the MFMA's internal K order does not matter. A chunk is 16 granules of 16
// bytes per row; MFMA s of the chunk takes granules 4s..4s+3, granule 4s+q in
// lane group q = lane/16. A weight load instruction therefore reads 64
// contiguous bytes of each of its 16 rows (4 lanes per row), which keeps the
// number of cache lines each load touches low.
#include <float.h>

#include <algorithm>
#include <cmath>
#include <type_traits>
#include <utility>

#include "gemm_tile.h"

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

// NW wavefronts per workgroup (4 or 8); with 8, two wavefronts share each
// SIMD, so one can issue MFMAs while the other waits on memory.
template <Elem EL, Epi EPI, int BM, int PD, int APD, bool SMAJOR, bool ASPLIT, int NW = 4>
__global__ __launch_bounds__(NW * 64, ((BM <= 32 || NW == 8) ? 2 : 1)) void gemm_kernel(GemmArgs a, int n_tiles) {
    constexpr int NT = NW * 64;                        // threads per workgroup
    constexpr int HC = NW * 32;                        // SWIGLU: h columns per tile
    constexpr int PC = NW * 64;                        // PLAIN: output columns per tile
    using T = Tr<EL>;
    constexpr int EB = T::kElemBytes;
    constexpr int RUNG = T::kRunG;
    constexpr int ROWG = T::kRowG;
    constexpr int ROWB = ROWG * 16;                    // LDS bytes per tile row
    constexpr int NRF = BM / 16;                       // 16-row blocks
    constexpr int ROWS_PER_PASS = NT / ROWG;           // A rows loaded per pass
    constexpr int PASSES = BM / ROWS_PER_PASS;
    constexpr int NB = PD + 1;                         // B register buffers
    constexpr int U = (NB % 2 == 0) ? NB : 2 * NB;     // unroll: every ring index static
    static_assert(BM % ROWS_PER_PASS == 0, "tile rows");
    static_assert(APD == 1 || APD == 2, "A prefetch distance");
    static_assert(!ASPLIT || APD == 1, "split A staging is one chunk ahead");

    // Two A-tile buffers of BM x ROWB bytes (dynamic: 128 KB at BM = 256).
    extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
    unsigned char* const s_a0 = s_dyn;
    unsigned char* const s_a1 = s_dyn + BM * ROWB;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;

    // ---- tile lookup -----------------------------------------------------
    Tile tl;
    if (!find_tile(a, n_tiles, BM, tl)) return;
    const int g = tl.g, ks = tl.ks, nt = tl.nt;
    const bool shared = tl.shared;
    const int row0 = tl.row0, m0 = tl.m0, rows = tl.rows;
    const int KS = a.ksplit;
    const int nrf = (rows + 15) >> 4;
    const int K = a.K;
    const int nch_all = K / T::kChunk;
    const int c_begin = (nch_all * ks) / KS;
    const int nch = (nch_all * (ks + 1)) / KS - c_begin;

    // ---- B (weights): per-lane pointers of the 4 column fragments ----------
    const unsigned char* Bg = shared ? static_cast<const unsigned char*>(a.B_shared)
                                     : static_cast<const unsigned char*>(a.B) + static_cast<int64_t>(g) * a.b_stride * EB;
    // Per-lane byte offsets of the 4 fragments' rows (an expert's weight
    // matrix is < 4 GiB, so 32 bits suffice and save VGPRs).
    const unsigned char* const Bb = Bg + static_cast<int64_t>(c_begin) * ROWB;
    uint32_t boff[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        int brow;
        if constexpr (EPI == Epi::SWIGLU) {
            int col = nt * HC + wave * 32 + 16 * (f & 1) + lr;
            col = col < a.inter ? col : a.inter - 1;   // column tail: valid row, result dropped
            brow = (f < 2) ? col : a.inter + col;
        } else {
            brow = nt * PC + wave * 64 + 16 * f + lr;
            brow = brow < a.N ? brow : a.N - 1;        // column tail: valid row, result dropped
        }
        boff[f] = static_cast<uint32_t>(brow) * static_cast<uint32_t>(K * EB) + lq * 16;
    }

    // ---- A (activations): per-thread row sources for the LDS fill ----------
    const int aj = tid % ROWG;                         // granule within the row
    const int ar = tid / ROWG;                         // first row of this thread
    const unsigned char* Abase = static_cast<const unsigned char*>(shared ? a.A_shared : a.A) + aj * 16 +
                                 static_cast<int64_t>(c_begin) * ROWB;
    // Byte offset of each A row this thread fills (an activation matrix is
    // < 4 GiB, so 32 bits suffice and save VGPRs).
    uint32_t aoff[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        int r = ar + i * ROWS_PER_PASS;
        r = r < rows ? r : rows - 1;                   // rows past the end: a valid row, unused
        uint32_t src_row;
        if (shared) src_row = m0 + r;
        else if (a.gather) src_row = static_cast<uint32_t>(a.perm[row0 + m0 + r] / a.topk);
        else src_row = row0 + m0 + r;
        aoff[i] = src_row * static_cast<uint32_t>(K * EB);
    }
    // LDS layout of the A tile: row r holds its 16-byte granules permuted by
    // XOR with r % 16, which makes both the tile fill (a wavefront writes 4
    // rows) and the fragment reads (16 rows, 4 adjacent granules per row)
    // conflict-free on gfx950's LDS (measured with the bank-conflict counter).
    auto swz = [](int r) { return r & 15; };
    // LDS store offset (row ar, swizzled granule); pass i adds i*ROWS_PER_PASS rows.
    const int a_st = ar * ROWB + ((aj ^ swz(ar & 15)) * 16);
    // LDS read offsets for sub-run s of this lane (row lr of each 16-row block).
    int a_ld[RUNG];
#pragma unroll
    for (int s = 0; s < RUNG; ++s) a_ld[s] = lr * ROWB + (((s * 4 + lq) ^ swz(lr)) * 16);

    f32x4 acc[NRF][4];
#pragma unroll
    for (int i = 0; i < NRF; ++i)
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    vec16 breg[SMAJOR ? 1 : NB][4][RUNG];
    vec16 areg[APD][PASSES];

    auto load_b = [&](vec16 (&dst)[4][RUNG], int c) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int s = 0; s < RUNG; ++s) dst[f][s] = ld16(Bb + boff[f] + static_cast<int64_t>(c) * ROWB + s * 64);
    };
    // Activation rows of passes [P0, P1) of chunk c: global -> VGPR, VGPR -> LDS.
    auto load_a = [&](vec16 (&dst)[PASSES], int c, auto p0, auto p1) __attribute__((always_inline)) {
#pragma unroll
        for (int i = decltype(p0)::value; i < decltype(p1)::value; ++i)
            dst[i] = ld16(Abase + aoff[i] + static_cast<int64_t>(c) * ROWB);
    };
    auto store_a = [&](const vec16 (&src)[PASSES], int buf, auto p0, auto p1) __attribute__((always_inline)) {
        unsigned char* dst = buf ? s_a1 : s_a0;
#pragma unroll
        for (int i = decltype(p0)::value; i < decltype(p1)::value; ++i)
            st16(dst + a_st + i * ROWS_PER_PASS * ROWB, src[i]);
    };
    using P0 = std::integral_constant<int, 0>;
    using PH = std::integral_constant<int, PASSES / 2>;
    using PE = std::integral_constant<int, PASSES>;
    // One chunk of MFMAs. The A fragments of 16-row block i+1 are read from
    // LDS before the 4*RUNG MFMAs of block i are issued, so LDS latency hides
    // behind matrix work; blocks past the tile's real rows are skipped.
    auto compute = [&](const vec16 (&b)[4][RUNG], int buf, auto&& mid) __attribute__((always_inline)) {
        const unsigned char* src = buf ? s_a1 : s_a0;
        vec16 af[2][RUNG];
#pragma unroll
        for (int s = 0; s < RUNG; ++s) af[0][s] = ld16(src + a_ld[s]);
#pragma unroll
        for (int i = 0; i < NRF; ++i) {
            if (i == NRF / 2) mid();
            // block 0 always has rows: its MFMAs (and the waits for this
            // chunk's weights) are unconditional
            if (i == 0 || i < nrf) {
                if (i + 1 < NRF) {
#pragma unroll
                    for (int s = 0; s < RUNG; ++s) af[(i + 1) & 1][s] = ld16(src + (i + 1) * 16 * ROWB + a_ld[s]);
                }
                // keep the next block's LDS reads ahead of this block's MFMAs
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int s = 0; s < RUNG; ++s)
#pragma unroll
                    for (int f = 0; f < 4; ++f) mfma_granule<EL>(af[i & 1][s], b[f][s], acc[i][f]);
            }
        }
    };

    // ---- main loop ---------------------------------------------------------
    // Every load is issued unconditionally (past the last chunk the index is
    // clamped and the data unused): conditional loads would make the
    // compiler's wait-count insertion drain all outstanding loads before each
    // chunk's first MFMA. The steady-state loop is straight-line; the last
    // (nch mod U) chunks run in a guarded remainder.
    // Chunk c's activations: global -> VGPR APD chunks ahead, VGPR -> LDS at
    // the end of chunk c-1, one barrier per chunk.
    const int last = nch - 1;
    if constexpr (!SMAJOR) {
        // Chunk c's weights are loaded PD chunks ahead
        // into a ring of VGPR buffers, so several chunks per wavefront are in
        // flight; loads are issued oldest-needed first.
        auto step = [&](auto uc, int c) __attribute__((always_inline)) {
            constexpr int u = decltype(uc)::value;
            if constexpr (ASPLIT) {
                // Halves: rows of the first half are stored mid-chunk, which
                // frees their VGPRs for the second half's loads.
                load_a(areg[0], c + 1 <= last ? c + 1 : last, P0{}, PH{});
                load_b(breg[(u + PD) % NB], min(c + PD, last));
                compute(breg[u % NB], u & 1, [&]() __attribute__((always_inline)) {
                    store_a(areg[0], (u + 1) & 1, P0{}, PH{});
                    load_a(areg[0], c + 1 <= last ? c + 1 : last, PH{}, PE{});
                });
                store_a(areg[0], (u + 1) & 1, PH{}, PE{});
            } else {
                load_a(areg[u % APD], min(c + APD, last), P0{}, PE{});
                load_b(breg[(u + PD) % NB], min(c + PD, last));
                compute(breg[u % NB], u & 1, [] {});
                store_a(areg[(u + 1) % APD], (u + 1) & 1, P0{}, PE{});
            }
            __syncthreads();
        };
        if (nch > 0) {
#pragma unroll
            for (int p = 0; p < APD; ++p) load_a(areg[p], min(p, last), P0{}, PE{});
#pragma unroll
            for (int p = 0; p < PD; ++p) load_b(breg[p], min(p, last));
            store_a(areg[0], 0, P0{}, PE{});
            __syncthreads();
        }
        int c = 0;
        for (; c + U <= nch; c += U) {
            [&]<int... I>(std::integer_sequence<int, I...>) {
                (step(std::integral_constant<int, I>{}, c + I), ...);
            }(std::make_integer_sequence<int, U>{});
        }
        [&]<int... I>(std::integer_sequence<int, I...>) {
            ((c + I < nch ? step(std::integral_constant<int, I>{}, c + I) : void()), ...);
        }(std::make_integer_sequence<int, U>{});
    } else {
        // Compute-bound tiles: one VGPR buffer of weights, consumed sub-run by
        // sub-run (s-major); once sub-run s of chunk c has fed its MFMAs, sub-
        // run s of chunk c+1 is loaded into the same registers, a full chunk
        // of MFMA time ahead of its use. A fragments are read from LDS one
        // step ahead of their MFMAs.
        vec16 (&b)[4][RUNG] = breg[0];
        auto step = [&](auto uc, int c) __attribute__((always_inline)) {
            constexpr int u = decltype(uc)::value;
            load_a(areg[u % APD], min(c + APD, last), P0{}, PE{});
            const unsigned char* src = (u & 1) ? s_a1 : s_a0;
            const int64_t nb = static_cast<int64_t>(min(c + 1, last)) * ROWB;
            vec16 af[2];
            af[0] = ld16(src + a_ld[0]);
#pragma unroll
            for (int s = 0; s < RUNG; ++s) {
#pragma unroll
                for (int i = 0; i < NRF; ++i) {
                    const int idx = s * NRF + i;
                    if (idx + 1 < RUNG * NRF) {
                        const int ni = (idx + 1) % NRF, ns = (idx + 1) / NRF;
                        af[(idx + 1) & 1] = ld16(src + ni * 16 * ROWB + a_ld[ns]);
                    }
                    if (i == 0 || i < nrf) {
#pragma unroll
                        for (int f = 0; f < 4; ++f) mfma_granule<EL>(af[idx & 1], b[f][s], acc[i][f]);
                    }
                }
#pragma unroll
                for (int f = 0; f < 4; ++f) b[f][s] = ld16(Bb + boff[f] + nb + s * 64);
            }
            store_a(areg[(u + 1) % APD], (u + 1) & 1, P0{}, PE{});
            __syncthreads();
        };
        if (nch > 0) {
#pragma unroll
            for (int p = 0; p < APD; ++p) load_a(areg[p], min(p, last), P0{}, PE{});
            load_b(b, 0);
            store_a(areg[0], 0, P0{}, PE{});
            __syncthreads();
        }
        constexpr int U2 = 2;
        int c = 0;
        for (; c + U2 <= nch; c += U2) {
            step(std::integral_constant<int, 0>{}, c);
            step(std::integral_constant<int, 1>{}, c + 1);
        }
        if (c < nch) step(std::integral_constant<int, 0>{}, c);
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
                    const int col = nt * HC + wave * 32 + 16 * f + lr;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int r = i * 16 + lq * 4 + v;
                        if (r < rows && col < a.N) {
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
                    const int col = nt * PC + wave * 64 + 16 * f + lr;
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
        // The slices' partial sums are loaded 8 at a time before any is
        // added, so their memory latencies overlap (past the last slice the
        // index is clamped and the value unused); they are added in slice
        // order, as a plain loop over the slices would.
        float v[4];
        for (int s0 = 0; s0 < a.ksplit; s0 += 8) {
            vec16 p[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) p[q] = ld16(a.partial + min(s0 + q, a.ksplit - 1) * stride + i);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (s0 + q < a.ksplit) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = s0 + q == 0 ? __uint_as_float(p[q].w[j]) : v[j] + __uint_as_float(p[q].w[j]);
                }
            }
        }
        if (a.bias) {
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] += a.bias[(i + j) % a.ldc];
        }
        st16(static_cast<float*>(a.C) + i,
             vec16{{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])}});
    }
}

// m-tile prefix over the groups: sched[g] = sum_{g' < g} ceil(rows_g' / bm);
// with splits, the XCD item ranges of each launch (XcdSplit). Items are
// ordered group by group, and within a group column tile by column tile with
// the m-tiles fastest (find_tile); an item of m-tile j costs the 32-row
// blocks of that tile plus cost_q / 4 blocks.
__global__ __launch_bounds__(kThreads) void schedule_kernel(GemmArgs a, int bm, int32_t* sched, XcdSplit sp0,
                                                            XcdSplit sp1, int n_splits) {
    constexpr int kMaxG = 4 * kThreads + 4;
    __shared__ int s_v[kMaxG];
    __shared__ int s_part[kThreads];
    __shared__ int s_blk[kMaxG];              // blocks with data over a group's m-tiles
    __shared__ long long s_w[kMaxG + 1];      // work prefix over the groups
    __shared__ long long s_wpart[kThreads];
    __shared__ long long s_wlast;
    __shared__ int s_b[8];
    const int n_groups = a.n_local + a.has_shared;
    for (int g = threadIdx.x; g < n_groups; g += kThreads) {
        int rows = a.T;
        if (!(a.has_shared && g == a.n_local) && a.offsets) rows = a.offsets[g + 1] - a.offsets[g];
        const int mt = (rows + bm - 1) / bm;
        s_v[g] = mt;
        // balanced split (find_tile): m-tiles of tr rows, tr a multiple of
        // 32, the last one the remainder (never empty, since tr <= bm)
        int blk = 0;
        if (mt > 0) {
            const int tr = min(bm, ((rows + mt - 1) / mt + 31) & ~31);
            blk = (mt - 1) * (tr / 32) + (rows - (mt - 1) * tr + 31) / 32;
        }
        s_blk[g] = blk;
    }
    __syncthreads();
    if (threadIdx.x == 0) s_part[0] = s_v[n_groups - 1];
    __syncthreads();
    const int last = s_part[0];
    __syncthreads();
    block_exclusive_scan<kThreads>(s_v, n_groups, s_part);
    for (int g = threadIdx.x; g < n_groups; g += kThreads) sched[g] = s_v[g];
    const int total_mt = s_v[n_groups - 1] + last;
    if (threadIdx.x == 0) sched[n_groups] = total_mt;
    for (int i = 0; i < n_splits; ++i) {
        const XcdSplit sp = i == 0 ? sp0 : sp1;
        // work of group g: n_tiles columns of (4 x its blocks + cost_q x its m-tiles)
        for (int g = threadIdx.x; g < n_groups; g += kThreads) {
            const int mt = (g + 1 < n_groups ? s_v[g + 1] : total_mt) - s_v[g];
            s_w[g] = static_cast<long long>(sp.n_tiles) * (4LL * s_blk[g] + static_cast<long long>(sp.cost_q) * mt);
        }
        __syncthreads();
        if (threadIdx.x == 0) s_wlast = s_w[n_groups - 1];
        __syncthreads();
        block_exclusive_scan<kThreads>(s_w, n_groups, s_wpart);
        const long long W = s_w[n_groups - 1] + s_wlast;
        // XCD x (1..7) starts at the item where x / 8 of the work is done
        if (threadIdx.x >= 1 && threadIdx.x < 8) {
            const long long t = W * threadIdx.x / 8;
            long long item = 0;
            if (t < W) {
                int lo = 0, hi = n_groups;                 // s_w[lo] <= t < s_w[hi] (s_w[n_groups] = W)
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (s_w[mid] <= t) lo = mid; else hi = mid;
                }
                const int mt = (lo + 1 < n_groups ? s_v[lo + 1] : total_mt) - s_v[lo];
                const long long colw = 4LL * s_blk[lo] + static_cast<long long>(sp.cost_q) * mt;   // > 0
                const long long rem = t - s_w[lo];
                const long long c = rem / colw;            // column tile
                const long long j = (rem - c * colw) * mt / colw;   // m-tile within it (pro rata)
                item = static_cast<long long>(s_v[lo]) * sp.n_tiles + c * mt + j;
            } else {
                item = static_cast<long long>(total_mt) * sp.n_tiles;
            }
            s_b[threadIdx.x] = static_cast<int>(item);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            // monotone, range x within x * cap, then every range at most cap
            // items: with 8 cap >= the item count every item keeps a slot
            const int total = total_mt * sp.n_tiles;
            int b[9];
            b[0] = 0;
            b[8] = total;
            for (int x = 1; x < 8; ++x) {
                int v = min(max(s_b[x], 0), total);
                v = static_cast<int>(min(static_cast<long long>(v), static_cast<long long>(x) * sp.cap));
                b[x] = max(v, b[x - 1]);
            }
            for (int x = 7; x >= 1; --x) b[x] = max(b[x], b[x + 1] - sp.cap);
            for (int x = 0; x < 9; ++x) sp.out[x] = b[x];
        }
        __syncthreads();
    }
}

// The items of up to two launches on the schedule as tiles (find_tile's
// arithmetic with the balanced row split, ksplit 1): table i gets entry L for
// every item L below launch i's item count and cap i. One thread per item.
__global__ __launch_bounds__(kThreads) void tile_table_kernel(GemmArgs a, int bm, int n0, int n1, int cap0, int cap1,
                                                              int4* t0, int4* t1) {
    const int n_groups = a.n_local + a.has_shared;
    const int m_total = a.sched[n_groups];
    const int L = static_cast<int>(blockIdx.x) * kThreads + static_cast<int>(threadIdx.x);
    for (int i = 0; i < 2; ++i) {
        const int n_tiles = i ? n1 : n0, cap = i ? cap1 : cap0;
        int4* tab = i ? t1 : t0;
        if (!tab || L >= m_total * n_tiles || L >= cap) continue;
        int lo = 0, hi = n_groups;                     // sched[lo]*n_tiles <= L < sched[hi]*n_tiles
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.sched[mid] * n_tiles <= L) lo = mid; else hi = mid;
        }
        const int g = lo, mt_begin = a.sched[g], mt_count = a.sched[g + 1] - mt_begin;
        const int local = L - mt_begin * n_tiles;
        const int nt = local / mt_count, mt = local - nt * mt_count;
        int rows_g = a.T, row0 = 0;
        if (!(a.has_shared && g == a.n_local) && a.offsets) {
            row0 = a.offsets[g];
            rows_g = a.offsets[g + 1] - row0;
        }
        const int tr = min(bm, ((rows_g + mt_count - 1) / mt_count + 31) & ~31);
        const int m0 = mt * tr;
        tab[L] = int4{g | (nt << 16), row0, m0, min(tr, rows_g - m0)};
    }
}

template <Elem EL, Epi EPI, int BM, int PD, int APD, bool SMAJOR = false, bool ASPLIT = false, int NW = 4>
void launch_one(const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    constexpr size_t lds = 2 * static_cast<size_t>(BM) * Tr<EL>::kRowG * 16;
    if constexpr (lds > 65536) {
        static std::atomic<int> lds_set[kMaxDevices];
        (void)ensure_dynamic_lds(reinterpret_cast<const void*>(&gemm_kernel<EL, EPI, BM, PD, APD, SMAJOR, ASPLIT, NW>),
                                 static_cast<int>(lds), lds_set);
    }
    hipLaunchKernelGGL((gemm_kernel<EL, EPI, BM, PD, APD, SMAJOR, ASPLIT, NW>), dim3(static_cast<unsigned>(p.grid)), dim3(NW * 64),
                       lds, s, a, p.n_tiles);
}

template <Elem EL, Epi EPI>
hipError_t launch_bm(GemmArgs a, const GemmPlan& p, hipStream_t s) {
    a.ksplit = p.ksplit < 1 ? 1 : p.ksplit;
    if (p.nw == 8) {
        if constexpr (EL == Elem::BF16) {
            if (p.smajor && p.bm == 128) launch_one<EL, EPI, 128, 1, 1, true, false, 8>(a, p, s);
            else if (p.smajor && p.bm == 96) launch_one<EL, EPI, 96, 1, 1, true, false, 8>(a, p, s);
            else if (!p.smajor && p.bm == 32) launch_one<EL, EPI, 32, 1, 2, false, false, 8>(a, p, s);
            else return hipErrorInvalidValue;
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    if (p.smajor) return hipErrorInvalidValue;
    switch (p.bm) {
        case 32: launch_one<EL, EPI, 32, 1, 2>(a, p, s); break;
        case 64: launch_one<EL, EPI, 64, 1, 2>(a, p, s); break;
        case 96:
            if constexpr (EL == Elem::BF16) {
                launch_one<EL, EPI, 96, 1, 2>(a, p, s);
                break;
            }
            return hipErrorInvalidValue;
        case 128: launch_one<EL, EPI, 128, 1, 2>(a, p, s); break;
        case 192:
            if constexpr (EL == Elem::BF16) {
                launch_one<EL, EPI, 192, 1, 1, false, true>(a, p, s);
                break;
            }
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

GemmPlan plan_gemm(Elem e, Epi epi, int64_t rows_upper, int n_groups, int64_t expected_rows_per_group, int N) {
    GemmPlan p;
    p.nw = 4;
    p.smajor = 0;
    p.big = 0;
    p.ksplit = 1;
    auto cols = [&](int nw) { return (epi == Epi::SWIGLU ? 32 : 64) * nw; };
    const double m = static_cast<double>(expected_rows_per_group);
    // Hundreds of rows per group and enough tiles to fill the GPU: 256 x 256
    // tiles through the LDS pipeline of gemm_big.hip.
    if (e == Elem::BF16 && m >= 256) {
        const GemmPlan big = plan_gemm_big(epi, rows_upper, n_groups, N);
        if ((rows_upper / 256) * big.n_tiles >= 512) return big;
    }
    if (m >= 128) {
        // Compute-bound shapes: 128-row tiles on 8 wavefronts (two per SIMD,
        // weights consumed sub-run by sub-run), unless that leaves fewer than
        // 64 workgroups. The 8-wavefront tile fits two wavefronts per SIMD, so
        // the shared expert of a decode batch shares CUs with the routed
        // experts' bandwidth-bound tiles running beside it (measured on the
        // EP8 decode share: 0.97 -> 0.92 ms per layer).
        p.bm = 128;
        if (e == Elem::BF16 && (epi == Epi::PLAIN || N % cols(8) == 0) &&
            (rows_upper / 128) * ((N + cols(8) - 1) / cols(8)) >= 64) {
            p.nw = 8;
            p.smajor = 1;
        }
    } else {
        // Bandwidth-bound shapes: one m-tile should cover nearly every group
        // (the expected count plus three standard deviations of a Poisson
        // count), because a second m-tile streams the same weights again.
        const double need = m + 3.0 * std::sqrt(m);
        p.bm = need <= 32 ? 32 : need <= 64 ? 64 : (need <= 96 && e == Elem::BF16) ? 96 : 128;
        // two wavefronts per SIMD (for SwiGLU only when 8 x 32 h columns tile N)
        if (e == Elem::BF16 && p.bm == 32 && (epi == Epi::PLAIN || N % cols(8) == 0)) p.nw = 8;
        if (e == Elem::BF16 && p.bm == 96 && epi == Epi::PLAIN) {
            p.nw = 8;
            p.smajor = 1;
        }
    }
    p.n_tiles = (N + cols(p.nw) - 1) / cols(p.nw);
    // sum_g ceil(rows_g / bm) <= rows_upper / bm + n_groups
    const int64_t m_tiles = rows_upper / p.bm + n_groups;
    p.grid = ((m_tiles * p.n_tiles + 7) / 8) * 8;
    return p;
}

GemmPlan plan_dense_splitk(int64_t T, int N, int K, int chunk) {
    GemmPlan p;
    p.nw = 4;
    p.smajor = 0;
    p.big = 0;
    // Row tile and K split by batch size (measured on the 7168 x 256 router:
    // small batches want many thin slices, large ones few wide tiles, since
    // every m-tile re-reads the weight from L2 and every slice adds a
    // partial-sum pass).
    int ks_max;
    if (T <= 1024) { p.bm = 32; ks_max = 16; }
    else if (T <= 4096) { p.bm = 64; ks_max = 8; }
    else if (T <= 8192) { p.bm = 128; ks_max = 4; }
    else { p.bm = 128; ks_max = 2; }
    p.n_tiles = (N + 255) / 256;
    const int64_t tiles = (T + p.bm - 1) / p.bm * p.n_tiles;
    const int nch = K / chunk;
    // each slice at least 3 chunks long; partial sums need N % 4 == 0
    int ks = 1;
    while (N % 4 == 0 && ks < ks_max && nch / (ks * 2) >= 3) ks *= 2;
    p.ksplit = ks;
    p.grid = ((tiles * ks + 7) / 8) * 8;
    return p;
}

int64_t splitk_partial_rows_upto(int64_t T, int N, int K, int chunk) {
    // ksplit * rows grows with T between the row-count breakpoints of
    // plan_dense_splitk and can drop just past one, so take the largest of T
    // and each breakpoint below it
    auto rows = [&](int64_t t) -> int64_t {
        const GemmPlan p = plan_dense_splitk(t, N, K, chunk);
        return p.ksplit > 1 ? p.ksplit * t : 0;
    };
    int64_t m = rows(T);
    for (const int64_t t : {int64_t{1024}, int64_t{4096}, int64_t{8192}})
        if (t < T) m = std::max(m, rows(t));
    return m;
}

hipError_t launch_splitk_reduce(const GemmArgs& a, int ksplit, hipStream_t s) {
    if (ksplit <= 1) return hipSuccess;
    const int64_t n4 = (static_cast<int64_t>(a.T) * a.ldc + 3) / 4;
    const int64_t blocks = std::min<int64_t>((n4 + kThreads - 1) / kThreads, 4096);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_schedule(const GemmArgs& a, int bm, int32_t* sched, hipStream_t s, const XcdSplit* splits,
                           int n_splits) {
    if (n_splits < 0 || n_splits > 2 || (n_splits > 0 && !splits)) return hipErrorInvalidValue;
    XcdSplit sp[2] = {};
    for (int i = 0; i < n_splits; ++i) {
        if (splits[i].n_tiles <= 0 || splits[i].cap <= 0 || splits[i].cost_q < 0 || !splits[i].out)
            return hipErrorInvalidValue;
        sp[i] = splits[i];
    }
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kThreads), 0, s, a, bm, sched, sp[0], sp[1], n_splits);
    return hipGetLastError();
}

hipError_t launch_tile_table(const GemmArgs& a, int bm, int n_launches, const int* n_tiles, const int* cap,
                             int4* const* tables, hipStream_t s) {
    if (n_launches < 1 || n_launches > 2 || !a.sched || bm <= 0) return hipErrorInvalidValue;
    int mx = 0;
    for (int i = 0; i < n_launches; ++i) {
        if (n_tiles[i] <= 0 || n_tiles[i] >= (1 << 15) || cap[i] < 0 || !tables[i]) return hipErrorInvalidValue;
        mx = std::max(mx, cap[i]);
    }
    if (mx == 0) return hipSuccess;
    const bool two = n_launches > 1;
    hipLaunchKernelGGL(tile_table_kernel, dim3(static_cast<unsigned>((mx + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       s, a, bm, n_tiles[0], two ? n_tiles[1] : 1, cap[0], two ? cap[1] : 0, tables[0],
                       two ? tables[1] : nullptr);
    return hipGetLastError();
}

hipError_t launch_gemm(Elem e, Epi epi, const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    if (p.grid == 0) return hipSuccess;
    if (p.big == 2) return e == Elem::BF16 ? launch_gemm_pf(epi, a, p, s) : hipErrorInvalidValue;
    if (p.big) return e == Elem::BF16 ? launch_gemm_big(epi, a, p, s) : hipErrorInvalidValue;
    if (e == Elem::BF16)
        return epi == Epi::SWIGLU ? launch_bm<Elem::BF16, Epi::SWIGLU>(a, p, s) : launch_bm<Elem::BF16, Epi::PLAIN>(a, p, s);
    if (e == Elem::F32)
        return epi == Epi::SWIGLU ? launch_bm<Elem::F32, Epi::SWIGLU>(a, p, s) : launch_bm<Elem::F32, Epi::PLAIN>(a, p, s);
    return hipErrorInvalidValue;
}

}  // namespace moe
