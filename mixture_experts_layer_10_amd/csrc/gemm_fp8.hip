// FP8 path: activation quantiser (K4) and the block-scaled grouped GEMM
// (K5/K6 with e4m3 operands) on gfx950 MFMA.
//
// What it computes: Perplexity "Lower latency and higher throughput with
// multi-node DeepSeek deployment", section "Quantization": weights carry one
// static scale per 128x128 block, activations one dynamic scale per 1x128
// vector computed online; for an (M, K) x (K, N) product the activation scales
// are (M, K/128) and the weight scales (K/128, N/128), and the SiLU kernel
// quantises its output per 128-element block. Formats: OCP E4M3FN (bias 7,
// largest finite value 448), round to nearest even; a block's scale is
// amax / 448 and its codes are e4m3(v * (448 / amax)), an all-zero block gets
// scale 1 and zero codes.
//
// GEMM structure: as the bf16 kernel (weights streamed into VGPRs, gathered
// activation tile in LDS, tiles dealt per XCD), with a K chunk of 128 = one
// scale block: each 16x16 output fragment takes one
// v_mfma_scale_f32_16x16x128_f8f6f4 per chunk (unit E8M0 scales) into a zeroed
// temporary, which is added to the fp32 accumulator times
// a_scale[row] * w_scale[column block] (the block dequantisation in fp32).
#include <float.h>

#include <type_traits>
#include <utility>

#include "gemm_tile.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 128;            // K per chunk = one scale block
constexpr int kRowB = 128;             // LDS bytes per A row per chunk
typedef int i32x8v __attribute__((ext_vector_type(8)));

// Two 16-byte loads straight into the 8 registers of one MFMA operand.
__device__ __forceinline__ i32x8v ld32(const void* lo, const void* hi) {
    typedef int i32x4v __attribute__((ext_vector_type(4)));
    const i32x4v a = *reinterpret_cast<const i32x4v*>(lo);
    const i32x4v b = *reinterpret_cast<const i32x4v*>(hi);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Two floats -> two e4m3 codes (round to nearest even, saturating at +-448),
// packed in the low 16 bits.
__device__ __forceinline__ uint32_t cvt2_e4m3(float a, float b) {
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}

// 448 / amax for a block with amax > 0; a block below about 2**-119, where
// the quotient overflows float32, takes the largest finite float32.
__device__ __forceinline__ float fp8_inv_scale(float amax) { return fminf(448.0f / amax, FLT_MAX); }

// ---- K4: per (row, 128-column block) quantisation of bf16 activations ------
// One workgroup per row; 16 lanes per 128-column block, 8 values per lane.
__global__ __launch_bounds__(kThreads) void quant_fp8_kernel(const uint16_t* x, uint8_t* q, float* scale,
                                                             int cols) {
    const int64_t row = blockIdx.x;
    const int nblk = cols / 128;
    const int sub = threadIdx.x & 15;
    for (int blk = threadIdx.x >> 4; blk < nblk; blk += kThreads / 16) {
        const int64_t off = row * cols + blk * 128 + sub * 8;
        const vec16 v = ld16(x + off);
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16_bits_to_f32(static_cast<uint16_t>(v.w[i] & 0xffffu));
            f[2 * i + 1] = bf16_bits_to_f32(static_cast<uint16_t>(v.w[i] >> 16));
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
        const bool nz = amax > 0.0f;
        const float inv = nz ? fp8_inv_scale(amax) : 0.0f;
        uint32_t lo = 0, hi = 0;
        if (nz) {
            lo = cvt2_e4m3(f[0] * inv, f[1] * inv) | (cvt2_e4m3(f[2] * inv, f[3] * inv) << 16);
            hi = cvt2_e4m3(f[4] * inv, f[5] * inv) | (cvt2_e4m3(f[6] * inv, f[7] * inv) << 16);
        }
        *reinterpret_cast<uint2*>(q + off) = make_uint2(lo, hi);
        if (sub == 0) scale[row * nblk + blk] = nz ? amax / 448.0f : 1.0f;
    }
}

// ---- K5/K6 in e4m3 -----------------------------------------------------------
// NW wavefronts (4 or 8) split the tile's 256 weight rows: each holds
// NF = 16 / NW fragments of 16 rows (SWIGLU: half gate, half up rows of the
// same h columns). With 8, the per-wavefront registers halve and two
// wavefronts share each SIMD, so one's dequantisation arithmetic overlaps the
// other's waits.
template <Epi EPI, int BM, int PD, int NW = 4>
__global__ __launch_bounds__(NW * 64, ((BM <= 32 || NW == 8) ? 2 : 1)) void gemm_fp8_kernel(GemmArgs a, int n_tiles) {
    constexpr int NT = NW * 64;
    constexpr int NF = 16 / NW;                        // 16-row fragments per wavefront
    constexpr int ROWG = kRowB / 16;                   // 8 granules per A row
    constexpr int NRF = BM / 16;
    constexpr int ROWS_PER_PASS = NT / ROWG;           // 32 or 64
    constexpr int PASSES = BM / ROWS_PER_PASS;
    constexpr int NB = PD + 1;
    constexpr int U = (NB % 2 == 0) ? NB : 2 * NB;
    constexpr int APD = 2;
    static_assert(BM % ROWS_PER_PASS == 0, "tile rows");

    __shared__ __attribute__((aligned(16))) unsigned char s_a[2][BM * kRowB];
    __shared__ __attribute__((aligned(16))) float s_sa[2][BM];      // activation scales of the chunk
    __shared__ float s_amax[NW][BM];                                // SwiGLU epilogue: per-wave row amax

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);      // wave-uniform: scalar scale loads
    const int lr = lane & 15, lq = lane >> 4;

    Tile tl;
    if (!find_tile(a, n_tiles, BM, tl, /*balanced=*/true)) return;
    const int g = tl.g, nt = tl.nt;
    const bool shared = tl.shared;
    const int row0 = tl.row0, m0 = tl.m0, rows = tl.rows;
    const int nrf = (rows + 15) >> 4;
    const int K = a.K;
    const int nch = K / kChunk;
    const int kblocks = K / 128;

    // ---- weights: e4m3 rows + fp32 scales per 128x128 block ---------------
    const int nb_rows = (EPI == Epi::SWIGLU ? 2 * a.inter : a.N) / 128;      // scale rows per expert
    const unsigned char* Bg = shared ? static_cast<const unsigned char*>(a.B_shared)
                                     : static_cast<const unsigned char*>(a.B) + static_cast<int64_t>(g) * a.b_stride;
    const float* Sg = shared ? static_cast<const float*>(a.B_scale_shared)
                             : static_cast<const float*>(a.B_scale) + static_cast<int64_t>(g) * nb_rows * kblocks;
    uint32_t boff[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        int brow;
        if constexpr (EPI == Epi::SWIGLU) {
            const int n0 = nt * 128 + wave * (128 / NW);
            brow = (f < NF / 2) ? n0 + 16 * f + lr : a.inter + n0 + 16 * (f - NF / 2) + lr;
        } else {
            brow = nt * 256 + wave * (256 / NW) + 16 * f + lr;
            brow = brow < a.N ? brow : a.N - 1;
        }
        boff[f] = static_cast<uint32_t>(brow) * static_cast<uint32_t>(K) + lq * 16;
    }
    // A wavefront's weight rows lie in one 128-row scale block per group
    // (SWIGLU: the gate rows and the up rows, the first and second half of
    // its fragments; PLAIN: all of them): its weight scales are wave-uniform,
    // one scalar load per group and chunk.
    constexpr int NG = EPI == Epi::SWIGLU ? 2 : 1;
    const float* bsc[NG];
    if constexpr (EPI == Epi::SWIGLU) {
        bsc[0] = Sg + nt * kblocks;
        bsc[1] = Sg + (a.inter / 128 + nt) * kblocks;
    } else {
        const int blk = min((nt * 256 + wave * (256 / NW)) / 128, a.N / 128 - 1);
        bsc[0] = Sg + blk * kblocks;
    }

    // ---- activations: gathered e4m3 rows and their per-block scales --------
    const int aj = tid % ROWG, ar = tid / ROWG;
    const unsigned char* Abase = static_cast<const unsigned char*>(shared ? a.A_shared : a.A) + aj * 16;
    const float* Ascale = static_cast<const float*>(shared ? a.A_scale_shared : a.A_scale);
    auto src_row = [&](int r) -> uint32_t {
        r = r < rows ? r : rows - 1;
        if (shared) return m0 + r;
        if (a.gather) return static_cast<uint32_t>(a.perm[row0 + m0 + r] / a.topk);
        return row0 + m0 + r;
    };
    uint32_t aoff[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) aoff[i] = src_row(ar + i * ROWS_PER_PASS) * static_cast<uint32_t>(K);
    const float* sa_src = tid < BM ? Ascale + static_cast<int64_t>(src_row(tid)) * kblocks : Ascale;
    static_assert(BM <= NT, "one activation-scale loader per tile row");
    // LDS: row r's granule j sits at j ^ (r & 7).
    const int a_st = ar * kRowB + ((aj ^ (ar & 7)) * 16);
    int a_ld[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) a_ld[s] = lr * kRowB + (((s * 4 + lq) ^ (lr & 7)) * 16);

    f32x4 acc[NRF][NF];
#pragma unroll
    for (int i = 0; i < NRF; ++i)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x8v breg[NB][NF];
    float bsreg[NB][NG];
    vec16 areg[APD][PASSES];
    float sareg[APD];
    const int last = nch - 1;

    auto load_b = [&](i32x8v (&dst)[NF], float (&ds)[NG], int c) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const unsigned char* p = Bg + boff[f] + static_cast<int64_t>(c) * kChunk;
            dst[f] = ld32(p, p + 64);
        }
#pragma unroll
        for (int q = 0; q < NG; ++q) ds[q] = bsc[q][c];
    };
    auto load_a = [&](vec16 (&dst)[PASSES], float& ds, int c) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < PASSES; ++i) dst[i] = ld16(Abase + aoff[i] + static_cast<int64_t>(c) * kChunk);
        ds = sa_src[c];
    };
    auto store_a = [&](const vec16 (&src)[PASSES], float ds, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < PASSES; ++i) st16(&s_a[buf][a_st + i * ROWS_PER_PASS * kRowB], src[i]);
        if (tid < BM) s_sa[buf][tid] = ds;
    };
    auto compute = [&](const i32x8v (&bv)[NF], const float (&bs)[NG], int buf) __attribute__((always_inline)) {
        const unsigned char* src = s_a[buf];
        i32x8v af[2];
        f32x4 sa[2];
        af[0] = ld32(src + a_ld[0], src + a_ld[1]);
        sa[0] = *reinterpret_cast<const f32x4*>(&s_sa[buf][4 * lq]);
#pragma unroll
        for (int i = 0; i < NRF; ++i) {
            if (i == 0 || i < nrf) {
                if (i + 1 < NRF) {
                    af[(i + 1) & 1] = ld32(src + (i + 1) * 16 * kRowB + a_ld[0], src + (i + 1) * 16 * kRowB + a_ld[1]);
                    sa[(i + 1) & 1] = *reinterpret_cast<const f32x4*>(&s_sa[buf][(i + 1) * 16 + 4 * lq]);
                }
                __builtin_amdgcn_sched_barrier(0);
                const i32x8v av = af[i & 1];
                f32x4 t[NF];
#pragma unroll
                for (int f = 0; f < NF; ++f)
                    t[f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv[f], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                           0, 127, 0, 127);
                // block dequantisation: acc += t * (a_scale[row] * w_scale)
                f32x4 cs[NG];
#pragma unroll
                for (int q = 0; q < NG; ++q) cs[q] = sa[i & 1] * bs[q];
#pragma unroll
                for (int f = 0; f < NF; ++f) acc[i][f] += t[f] * cs[NG == 2 ? f / (NF / 2) : 0];
            }
        }
    };

    // ---- main loop (branch-free steady state; see the bf16 kernel) --------
    auto step = [&](auto uc, int c) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        load_a(areg[u % APD], sareg[u % APD], min(c + APD, last));
        load_b(breg[(u + PD) % NB], bsreg[(u + PD) % NB], min(c + PD, last));
        compute(breg[u % NB], bsreg[u % NB], u & 1);
        store_a(areg[(u + 1) % APD], sareg[(u + 1) % APD], (u + 1) & 1);
        __syncthreads();
    };
    if (nch > 0) {
#pragma unroll
        for (int p = 0; p < APD; ++p) load_a(areg[p], sareg[p], min(p, last));
#pragma unroll
        for (int p = 0; p < PD; ++p) load_b(breg[p], bsreg[p], min(p, last));
        store_a(areg[0], sareg[0], 0);
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

    // ---- epilogue ------------------------------------------------------------
    const int64_t crow0 = shared ? m0 : static_cast<int64_t>(row0) + m0;
    if constexpr (EPI == Epi::SWIGLU) {
        // h = silu(g) * u in fp32, then e4m3 with one scale per (row, 128
        // columns): this tile's 128 h columns are exactly one scale block.
        float h[NRF][NF / 2][4];
#pragma unroll
        for (int i = 0; i < NRF; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float m = 0.0f;
#pragma unroll
                for (int f = 0; f < NF / 2; ++f) {
                    const float gv = acc[i][f][v], uv = acc[i][f + NF / 2][v];
                    h[i][f][v] = silu_mul(gv, uv);
                    m = fmaxf(m, fabsf(h[i][f][v]));
                }
#pragma unroll
                for (int s = 1; s < 16; s <<= 1) m = fmaxf(m, __shfl_xor(m, s, 16));
                if (lr == 0) s_amax[wave][i * 16 + lq * 4 + v] = m;
            }
        __syncthreads();
        uint8_t* Cq = static_cast<uint8_t*>(shared ? a.C_shared : a.C);
        float* Cs = static_cast<float*>(shared ? a.C_scale_shared : a.C_scale);
        const int nsb = a.N / 128;
#pragma unroll
        for (int i = 0; i < NRF; ++i) {
            if (i < nrf) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = i * 16 + lq * 4 + v;
                    float amax = s_amax[0][r];
#pragma unroll
                    for (int w = 1; w < NW; ++w) amax = fmaxf(amax, s_amax[w][r]);
                    const bool nz = amax > 0.0f;
                    const float inv = nz ? fp8_inv_scale(amax) : 0.0f;
                    if (r < rows) {
#pragma unroll
                        for (int f = 0; f < NF / 2; ++f) {
                            const int col = nt * 128 + wave * (128 / NW) + 16 * f + lr;
                            const uint32_t code = nz ? (cvt2_e4m3(h[i][f][v] * inv, 0.0f) & 0xffu) : 0u;
                            Cq[(crow0 + r) * a.ldc + col] = static_cast<uint8_t>(code);
                        }
                        if (wave == 0 && lr == 0) Cs[(crow0 + r) * nsb + nt] = nz ? amax / 448.0f : 1.0f;
                    }
                }
            }
        }
    } else {
        unsigned char* Cb = static_cast<unsigned char*>(shared ? a.C_shared : a.C);
#pragma unroll
        for (int i = 0; i < NRF; ++i) {
            if (i < nrf) {
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                    const int col = nt * 256 + wave * (256 / NW) + 16 * f + lr;
                    if (col < a.N) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int r = i * 16 + lq * 4 + v;
                            if (r < rows) {
                                const int64_t off = (crow0 + r) * a.ldc + col;
                                if (a.out_f32)
                                    reinterpret_cast<float*>(Cb)[off] = acc[i][f][v];
                                else
                                    reinterpret_cast<uint16_t*>(Cb)[off] = f32_to_bf16_bits(acc[i][f][v]);
                            }
                        }
                    }
                }
            }
        }
    }
}

// ---- compute-bound shapes: 256 x 256 tiles staged through LDS -------------
// For groups of a thousand rows and more (the shared expert at prefill-sized
// batches) the weights are reused by many row tiles and the product is bound
// by matrix throughput. The structure is the bf16 256 x 256 kernel's:
//  * 8 wavefronts as 2 (rows) x 4 (weight rows), each 128 x 64 as 16 x 16
//    fragments of v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales);
//  * both operands HBM/L2 -> LDS by direct loads, K = 128 per stage (one
//    128-byte line per row), two stages; the stage's 256 activation scales
//    ride along in 4-byte direct loads;
//  * one scale block per stage: the fragment's product is added to the
//    accumulator times a_scale[row] * w_scale[block] (the weight block of a
//    wavefront's gate, up or plain columns is uniform: scalar loads).
constexpr int kBigKB = 128;                         // K (bytes) per stage
constexpr int kBigRows = 256;
constexpr int kBigStageB = 2 * kBigRows * kBigKB + kBigRows * 4;   // A, B, A scales
constexpr int kBigStages = 2;

__device__ __forceinline__ int big_swz(int r) { return (r >> 1) & 7; }

template <Epi EPI>
__global__ __launch_bounds__(512, 1) void gemm_big_fp8_kernel(GemmArgs a, int n_tiles) {
    constexpr int NW = 8, NT = 512;
    constexpr int GRAN = kBigKB / 16;                  // 8 granules per row
    constexpr int LOADS = kBigRows * GRAN / NT;        // 4 direct loads per operand per stage
    constexpr int RPL = 64 / GRAN;                     // 8 rows per load instruction
    extern __shared__ __attribute__((aligned(16))) unsigned char s_ring[];
    __shared__ float s_amax[4][kBigRows];              // SWIGLU epilogue: per-wave-column row amax

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int lr = lane & 15, lq = lane >> 4;

    Tile tl;
    if (!find_tile(a, n_tiles, kBigRows, tl, /*balanced=*/true)) return;
    const int g = tl.g, nt = tl.nt;
    const bool shared = tl.shared;
    const int row0 = tl.row0, m0 = tl.m0, rows = tl.rows;
    const int K = a.K;
    const int nkb = K / kBigKB;
    const int last = nkb - 1;

    auto src_row = [&](int r) -> uint32_t {
        r = r < rows ? r : rows - 1;
        if (shared) return m0 + r;
        if (a.gather) return static_cast<uint32_t>(a.perm[row0 + m0 + r] / a.topk);
        return row0 + m0 + r;
    };
    // direct-load sources: instruction j of wavefront w fills tile rows
    // (8 j + w) * 8 + lane / 8, granule slot lane % 8, with the granule the
    // swizzle places there
    const int lrow = lane / GRAN;
    const unsigned char* Ag = static_cast<const unsigned char*>(shared ? a.A_shared : a.A);
    uint32_t aoff[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int rs = (NW * j + wave) * RPL + lrow;
        aoff[j] = src_row(rs) * static_cast<uint32_t>(K) + (((lane % GRAN) ^ big_swz(rs)) * 16);
    }
    const unsigned char* Bg = shared ? static_cast<const unsigned char*>(a.B_shared)
                                     : static_cast<const unsigned char*>(a.B) + static_cast<int64_t>(g) * a.b_stride;
    uint32_t boff[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int n = (NW * j + wave) * RPL + lrow;   // weight slot of the tile
        int brow;
        if constexpr (EPI == Epi::SWIGLU) {
            // slots [64 w, 64 w + 64): 32 gate rows, then the 32 up rows of the same h columns
            const int m = n & 63;
            int col = nt * 128 + (n >> 6) * 32 + (m & 31);
            col = col < a.inter ? col : a.inter - 1;
            brow = m < 32 ? col : a.inter + col;
        } else {
            brow = nt * 256 + n;
            brow = brow < a.N ? brow : a.N - 1;
        }
        boff[j] = static_cast<uint32_t>(brow) * static_cast<uint32_t>(K) + (((lane % GRAN) ^ big_swz(n)) * 16);
    }
    const int kblocks = K / 128;
    const float* Ascale = static_cast<const float*>(shared ? a.A_scale_shared : a.A_scale);
    const uint32_t sa_off = wave < 4 ? src_row(wave * 64 + lane) * static_cast<uint32_t>(kblocks) : 0u;
    // weight scales: one 128 x 128 block per wavefront and group
    const int nb_rows = (EPI == Epi::SWIGLU ? 2 * a.inter : a.N) / 128;
    const float* Sg = shared ? static_cast<const float*>(a.B_scale_shared)
                             : static_cast<const float*>(a.B_scale) + static_cast<int64_t>(g) * nb_rows * kblocks;
    const float* bsc0;
    const float* bsc1;
    if constexpr (EPI == Epi::SWIGLU) {
        bsc0 = Sg + nt * kblocks;
        bsc1 = Sg + (a.inter / 128 + nt) * kblocks;
    } else {
        bsc0 = bsc1 = Sg + min((nt * 256 + wn * 64) / 128, a.N / 128 - 1) * kblocks;
    }

    auto issue = [&](int kb, int slot) __attribute__((always_inline)) {
        unsigned char* sa = s_ring + slot * kBigStageB;
        unsigned char* sb = sa + kBigRows * kBigKB;
        float* ss = reinterpret_cast<float*>(sb + kBigRows * kBigKB);
        const uint32_t ko = static_cast<uint32_t>(kb) * kBigKB;
#pragma unroll
        for (int j = 0; j < LOADS; ++j)
            __builtin_amdgcn_global_load_lds(Ag + (aoff[j] + ko),
                                             (__attribute__((address_space(3))) void*)(sa + (NW * j + wave) * RPL * kBigKB),
                                             16, 0, 0);
#pragma unroll
        for (int j = 0; j < LOADS; ++j)
            __builtin_amdgcn_global_load_lds(Bg + (boff[j] + ko),
                                             (__attribute__((address_space(3))) void*)(sb + (NW * j + wave) * RPL * kBigKB),
                                             16, 0, 0);
        if (wave < 4)
            __builtin_amdgcn_global_load_lds(Ascale + (sa_off + kb),
                                             (__attribute__((address_space(3))) void*)(ss + wave * 64), 4, 0, 0);
    };
    auto sync = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0070);            // vmcnt 0, expcnt 7 (no wait), lgkmcnt 0
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // fragment reads: row r of a 16-row block, granules lq and 4 + lq
    int fo[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) fo[h] = lr * kBigKB + (((4 * h + lq) ^ big_swz(lr)) * 16);
    const int nrb = (rows + 15) >> 4;                  // 16-row blocks with data
    const int nbw = min(max(nrb - wm * 8, 0), 8);      // of this wavefront's 8 (uniform)

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    issue(0, 0);
    for (int kb = 0; kb < nkb; ++kb) {
        // stage kb has landed for every thread; stage kb - 1's slot is free
        sync();
        if (kb + 1 <= last) issue(kb + 1, (kb + 1) & 1);
        const unsigned char* st = s_ring + (kb & 1) * kBigStageB;
        const float* ss = reinterpret_cast<const float*>(st + 2 * kBigRows * kBigKB);
        const float sb0 = bsc0[kb], sb1 = bsc1[kb];
        i32x8v bfr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const unsigned char* p = st + kBigRows * kBigKB + (wn * 64 + j * 16) * kBigKB;
            bfr[j] = ld32(p + fo[0], p + fo[1]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i < nbw) {
                const unsigned char* p = st + (wm * 128 + i * 16) * kBigKB;
                const i32x8v af = ld32(p + fo[0], p + fo[1]);
                const f32x4 sa = *reinterpret_cast<const f32x4*>(ss + wm * 128 + i * 16 + 4 * lq);
                const f32x4 c0 = sa * sb0, c1 = sa * sb1;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bfr[j], f32x4{0.f, 0.f, 0.f, 0.f},
                                                                                  0, 0, 0, 127, 0, 127);
                    acc[i][j] += t * ((EPI == Epi::SWIGLU && j >= 2) ? c1 : c0);
                }
            }
        }
    }

    // ---- epilogue -----------------------------------------------------------
    // Outputs are staged in the (now idle) LDS ring as a row-major tile and
    // written as whole 16-byte pieces of rows: a lane's fragment values are
    // one column each, so direct stores would be 1-byte (e4m3 codes) or
    // 4-byte (fp32) writes spread over 16 rows per instruction. N and ldc are
    // multiples of 16 (checked at launch), so a piece is wholly inside the
    // output or wholly past its last column, and aligned.
    const int64_t crow0 = shared ? m0 : static_cast<int64_t>(row0) + m0;
    if constexpr (EPI == Epi::SWIGLU) {
        // h = silu(g) * u; the tile's 128 h columns are one 1x128 scale block:
        // row amax over this wavefront's 32 columns, then across the 4
        // wavefront columns in LDS
        float h[8][2][4];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float m = 0.0f;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float gv = acc[i][j][v], uv = acc[i][j + 2][v];
                    h[i][j][v] = silu_mul(gv, uv);
                    m = fmaxf(m, fabsf(h[i][j][v]));
                }
#pragma unroll
                for (int sft = 1; sft < 16; sft <<= 1) m = fmaxf(m, __shfl_xor(m, sft, 16));
                if (lr == 0) s_amax[wn][wm * 128 + i * 16 + 4 * lq + v] = m;
            }
        __syncthreads();                       // also: every fragment read of the ring is done
        uint8_t* Cq = static_cast<uint8_t*>(shared ? a.C_shared : a.C);
        float* Cs = static_cast<float*>(shared ? a.C_scale_shared : a.C_scale);
        const int nsb = a.N / 128;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i < nbw) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = wm * 128 + i * 16 + 4 * lq + v;
                    const float amax = fmaxf(fmaxf(s_amax[0][r], s_amax[1][r]), fmaxf(s_amax[2][r], s_amax[3][r]));
                    const bool nz = amax > 0.0f;
                    const float inv = nz ? fp8_inv_scale(amax) : 0.0f;
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        s_ring[r * 128 + wn * 32 + j * 16 + lr] =
                            static_cast<uint8_t>(nz ? (cvt2_e4m3(h[i][j][v] * inv, 0.0f) & 0xffu) : 0u);
                    if (r < rows && wn == 0 && lr == 0) Cs[(crow0 + r) * nsb + nt] = nz ? amax / 448.0f : 1.0f;
                }
            }
        }
        __syncthreads();
        for (int q = tid; q < rows * 8; q += NT) {
            const int r = q >> 3, col = nt * 128 + (q & 7) * 16;
            if (col < a.N) st16(Cq + (crow0 + r) * a.ldc + col, *reinterpret_cast<const vec16*>(s_ring + r * 128 + (q & 7) * 16));
        }
    } else {
        unsigned char* Cb = static_cast<unsigned char*>(shared ? a.C_shared : a.C);
        // bf16 outputs in one pass of the tile's 256 columns, fp32 in two of
        // 128 (128 KB of the ring each)
        auto epilogue = [&](auto f32_out) __attribute__((always_inline)) {
            constexpr bool F32 = decltype(f32_out)::value;
            constexpr int EB = F32 ? 4 : 2, PC = F32 ? 128 : 256, PRB = PC * EB, GPR = PRB / 16;
            auto pass = [&](auto pass_c) __attribute__((always_inline)) {
                constexpr int P = decltype(pass_c)::value;
                __syncthreads();               // fragment reads (or the previous pass's stores) are done
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (i < nbw) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int col = wn * 64 + j * 16 - P * PC;   // the fragment's first column in the pass
                            if (col >= 0 && col < PC) {                  // uniform: a fragment lies in one pass
#pragma unroll
                                for (int v = 0; v < 4; ++v) {
                                    unsigned char* row = s_ring + (wm * 128 + i * 16 + 4 * lq + v) * PRB;
                                    if constexpr (F32)
                                        reinterpret_cast<float*>(row)[col + lr] = acc[i][j][v];
                                    else
                                        reinterpret_cast<uint16_t*>(row)[col + lr] = f32_to_bf16_bits(acc[i][j][v]);
                                }
                            }
                        }
                    }
                }
                __syncthreads();
                const int c0 = nt * 256 + P * PC;
                for (int q = tid; q < rows * GPR; q += NT) {
                    const int r = q / GPR, gq = q % GPR;
                    const int col = c0 + gq * (16 / EB);
                    if (col < a.N)
                        st16(Cb + ((crow0 + r) * a.ldc + col) * EB, *reinterpret_cast<const vec16*>(s_ring + r * PRB + gq * 16));
                }
            };
            pass(std::integral_constant<int, 0>{});
            if constexpr (F32) pass(std::integral_constant<int, 1>{});
        };
        if (a.out_f32)
            epilogue(std::true_type{});
        else
            epilogue(std::false_type{});
    }
}

template <Epi EPI>
hipError_t launch_big_fp8(const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    constexpr int lds = kBigStages * kBigStageB;
    static_assert(lds >= 128 * 1024, "the epilogue stages 128 KB of outputs in the ring");
    if (a.N % 16 != 0 || a.ldc % 16 != 0) return hipErrorInvalidValue;
    static std::atomic<int> lds_set[kMaxDevices];
    const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&gemm_big_fp8_kernel<EPI>), lds, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_big_fp8_kernel<EPI>), dim3(static_cast<unsigned>(p.grid)), dim3(512), lds, s, a, p.n_tiles);
    return hipGetLastError();
}

template <Epi EPI>
hipError_t launch_fp8_bm(const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(p.grid));
    if (p.nw == 8) {
        if (p.bm != 64) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gemm_fp8_kernel<EPI, 64, 1, 8>), grid, dim3(512), 0, s, a, p.n_tiles);
        return hipGetLastError();
    }
    const dim3 block(kThreads);
    switch (p.bm) {
        case 32: hipLaunchKernelGGL((gemm_fp8_kernel<EPI, 32, 1>), grid, block, 0, s, a, p.n_tiles); break;
        case 64: hipLaunchKernelGGL((gemm_fp8_kernel<EPI, 64, 1>), grid, block, 0, s, a, p.n_tiles); break;
        case 128: hipLaunchKernelGGL((gemm_fp8_kernel<EPI, 128, 1>), grid, block, 0, s, a, p.n_tiles); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_fp8(const void* x_bf16, uint8_t* q, float* scale, int64_t rows, int cols, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_fp8_kernel, dim3(static_cast<unsigned>(rows)), dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(x_bf16), q, scale, cols);
    return hipGetLastError();
}

GemmPlan plan_gemm_fp8(Epi epi, int64_t rows_upper, int n_groups, int64_t expected_rows_per_group, int N) {
    GemmPlan p;
    p.nw = 4;
    p.smajor = 0;
    p.big = 0;
    p.ksplit = 1;
    // 64-row tiles unless groups are large: the weight streams dominate and
    // a 64-row tile keeps the dequantisation work per streamed byte low
    // (measured: 64 faster than 128 at ~50 rows per active expert).
    p.bm = expected_rows_per_group <= 32 ? 32 : expected_rows_per_group < 512 ? 64 : 128;
    if (p.bm == 64) p.nw = 8;                  // 8 wavefronts, two per SIMD (measured ~6% faster)
    const int cols = epi == Epi::SWIGLU ? 128 : 256;
    p.n_tiles = (N + cols - 1) / cols;
    const int64_t m_tiles = rows_upper / p.bm + n_groups;
    p.grid = ((m_tiles * p.n_tiles + 7) / 8) * 8;
    return p;
}

GemmPlan plan_gemm_fp8_big(Epi epi, int64_t rows_upper, int n_groups, int N) {
    GemmPlan p;
    p.bm = kBigRows;
    p.nw = 8;
    p.smajor = 0;
    p.big = 1;
    p.ksplit = 1;
    const int cols = epi == Epi::SWIGLU ? 128 : 256;
    p.n_tiles = (N + cols - 1) / cols;
    const int64_t m_tiles = rows_upper / kBigRows + n_groups;
    p.grid = ((m_tiles * p.n_tiles + 7) / 8) * 8;
    return p;
}

hipError_t launch_gemm_fp8(Epi epi, const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    if (p.grid == 0) return hipSuccess;
    GemmArgs b = a;
    b.ksplit = 1;
    if (p.big) return epi == Epi::SWIGLU ? launch_big_fp8<Epi::SWIGLU>(b, p, s) : launch_big_fp8<Epi::PLAIN>(b, p, s);
    return epi == Epi::SWIGLU ? launch_fp8_bm<Epi::SWIGLU>(b, p, s) : launch_fp8_bm<Epi::PLAIN>(b, p, s);
}

}  // namespace moe
