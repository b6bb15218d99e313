// FP4 path: MX activation quantiser and the grouped GEMM with FP4 (E2M1)
// expert weights and e4m3 activations, each with one power-of-two (E8M0)
// scale per 32 elements along K, on gfx950's scaled MFMA.
//
// What it computes: NVIDIA "Optimizing DeepSeek R1 throughput on Blackwell"
// runs DeepSeek R1 from a checkpoint whose MoE-layer weights are FP4 (section
// on the FP4 checkpoint: half the weight memory of FP8). The pages fix no
// encoding; this path takes the OCP microscaling one that gfx950's MFMA
// implements: E2M1 elements (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
// negatives) two to a byte, element 2i in the low nibble, and one E8M0 scale
// 2**(code - 127) per 32 consecutive elements of a weight row. Activations
// (x before the gate/up GEMM, h before the down GEMM) are e4m3 with the same
// 32-element power-of-two scales: X = floor(log2(max |v|)) - 8, clamped to
// [-127, 127] (an all-zero block takes -127), codes e4m3(v * 2**-X) rounded
// to nearest even and saturated at +-448.
//
// GEMM structure: the FP8 kernel's (weights streamed into VGPRs, gathered
// activation tile in LDS, tiles dealt per XCD), with a K chunk of 256 so that
// each weight row is read one whole 128-byte line per chunk. Every 16x16
// output fragment takes two v_mfma_scale_f32_16x16x128_f8f6f4 per chunk
// (A e4m3, B e2m1) that apply both block scales in the matrix core and
// accumulate straight into the fp32 accumulator: no dequantising arithmetic.
// Operand layout of that instruction (measured on the device): lane
// (q = lane / 16, r = lane % 16) holds, of row r, e4m3 bytes K = 16q..16q+15
// and 64+16q..64+16q+15, or E2M1 elements K = 32q..32q+31; its scale
// operand is the scale of K block q (K = 32q..32q+31) of row r.
#include <type_traits>
#include <utility>

#include "gemm_tile.h"

namespace moe {
namespace {

constexpr int kChunk = 256;            // K per chunk: two MFMA K-steps
constexpr int kRowA = 256;             // LDS bytes per A row per chunk
constexpr int kRowG = kRowA / 16;      // 16-byte granules per A row per chunk
constexpr int kBlk = 32;               // MX block (elements per scale)
typedef int i32x4v __attribute__((ext_vector_type(4)));

// Two floats -> two e4m3 codes (round to nearest even, saturating at +-448),
// packed in the low 16 bits.
__device__ __forceinline__ uint32_t cvt2_e4m3_sat(float a, float b) {
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}

// Shared exponent of a block with maximum magnitude m >= 0:
// floor(log2(m)) - 8 (the exponent field of a normal float), clamped at -127;
// zero and subnormal maxima give -127.
__device__ __forceinline__ int mx_exponent(float m) {
    const int e = static_cast<int>((__float_as_uint(m) >> 23) & 0xffu) - 127;
    return max(e - 8, -127);
}

// 2**-X as a float for X in [-127, 119] (always a normal number).
__device__ __forceinline__ float mx_inv_scale(int X) { return __uint_as_float(static_cast<uint32_t>(127 - X) << 23); }

// ---- x -> MX e4m3: one workgroup per row, 4 lanes per 32-column block ------
__global__ __launch_bounds__(256) void quant_mx_kernel(const uint16_t* x, uint8_t* q, uint8_t* scale, int cols) {
    const int64_t row = blockIdx.x;
    const int nblk = cols / kBlk;
    const int sub = threadIdx.x & 3;
    for (int blk = threadIdx.x >> 2; blk < nblk; blk += 64) {
        const int64_t off = row * cols + blk * kBlk + sub * 8;
        const vec16 v = ld16(x + off);
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16_bits_to_f32(static_cast<uint16_t>(v.w[i] & 0xffffu));
            f[2 * i + 1] = bf16_bits_to_f32(static_cast<uint16_t>(v.w[i] >> 16));
        }
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
        m = fmaxf(m, __shfl_xor(m, 1, 4));
        m = fmaxf(m, __shfl_xor(m, 2, 4));
        const int X = mx_exponent(m);
        const float inv = mx_inv_scale(X);
        const uint32_t lo = cvt2_e4m3_sat(f[0] * inv, f[1] * inv) | (cvt2_e4m3_sat(f[2] * inv, f[3] * inv) << 16);
        const uint32_t hi = cvt2_e4m3_sat(f[4] * inv, f[5] * inv) | (cvt2_e4m3_sat(f[6] * inv, f[7] * inv) << 16);
        *reinterpret_cast<uint2*>(q + off) = make_uint2(lo, hi);
        if (sub == 0) scale[row * nblk + blk] = static_cast<uint8_t>(X + 127);
    }
}

// ---- K5/K6 with FP4 weights ---------------------------------------------------
// NW wavefronts split the tile's 256 weight rows: each holds NF = 16 / NW
// fragments of 16 rows (SWIGLU: half gate, half up rows of the same h
// columns).
template <Epi EPI, int BM, int NW = 4>
__global__ __launch_bounds__(NW * 64, ((BM <= 32 || NW == 8) ? 2 : 1)) void gemm_mx_kernel(GemmArgs a, int n_tiles) {
    constexpr int NT = NW * 64;
    constexpr int NF = 16 / NW;                        // 16-row fragments per wavefront
    constexpr int NRF = BM / 16;
    constexpr int ROWS_PER_PASS = NT / kRowG;          // 16 or 32
    constexpr int PASSES = BM / ROWS_PER_PASS;
    constexpr int PD = 1;                              // weight chunks in flight beyond the current one
    constexpr int NB = PD + 1;
    constexpr int APD = 2;
    constexpr int U = 2;                               // steps per unrolled loop body (NB and 2 LDS buffers)
    static_assert(BM % ROWS_PER_PASS == 0, "tile rows");
    static_assert(BM <= NT, "one activation-scale loader per tile row");

    __shared__ __attribute__((aligned(16))) unsigned char s_a[2][BM * kRowA];
    __shared__ __attribute__((aligned(16))) uint2 s_sa[2][BM];     // 8 scale bytes per row per chunk
    constexpr int CPW = 16 * (NF / 2);                              // SWIGLU: h columns per wavefront
    constexpr int WPB = CPW >= kBlk ? 1 : kBlk / CPW;               // wavefronts per 32-column block
    __shared__ float s_amax[WPB > 1 ? NW : 1][WPB > 1 ? BM : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lq = lane >> 4;

    Tile tl;
    if (!find_tile(a, n_tiles, BM, tl, /*balanced=*/true)) return;
    const int g = tl.g, nt = tl.nt;
    const bool shared = tl.shared;
    const int row0 = tl.row0, m0 = tl.m0, rows = tl.rows;
    const int nrf = (rows + 15) >> 4;
    const int K = a.K;
    const int nch = K / kChunk;
    const int kb = K / kBlk;                           // scale bytes per row

    // ---- weights: packed E2M1 rows (K/2 bytes) and E8M0 scales (K/32 bytes)
    const int nb_rows = EPI == Epi::SWIGLU ? 2 * a.inter : a.N;
    const unsigned char* Bg = shared ? static_cast<const unsigned char*>(a.B_shared)
                                     : static_cast<const unsigned char*>(a.B) + static_cast<int64_t>(g) * a.b_stride;
    const unsigned char* Sg = shared ? static_cast<const unsigned char*>(a.B_scale_shared)
                                     : static_cast<const unsigned char*>(a.B_scale) +
                                           static_cast<int64_t>(g) * nb_rows * kb;
    uint32_t boff[NF], soff[NF];
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
        boff[f] = static_cast<uint32_t>(brow) * static_cast<uint32_t>(K / 2) + lq * 16;
        soff[f] = static_cast<uint32_t>(brow) * static_cast<uint32_t>(kb);
    }

    // ---- activations: gathered e4m3 rows and their scale bytes ------------
    const int aj = tid % kRowG, ar = tid / kRowG;
    const unsigned char* Abase = static_cast<const unsigned char*>(shared ? a.A_shared : a.A) + aj * 16;
    const unsigned char* Ascale = static_cast<const unsigned char*>(shared ? a.A_scale_shared : a.A_scale);
    auto src_row = [&](int r) -> uint32_t {
        r = r < rows ? r : rows - 1;
        if (shared) return m0 + r;
        if (a.gather) return static_cast<uint32_t>(a.perm[row0 + m0 + r] / a.topk);
        return row0 + m0 + r;
    };
    uint32_t aoff[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) aoff[i] = src_row(ar + i * ROWS_PER_PASS) * static_cast<uint32_t>(K);
    const unsigned char* sa_src = Ascale + (tid < BM ? static_cast<int64_t>(src_row(tid)) * kb : 0);
    // LDS: row r's granule j sits at j ^ (r & 15): the 16 rows of a fragment
    // read 16 different granule slots, so the 64 lanes' reads spread over all banks.
    const int a_st = ar * kRowA + ((aj ^ (ar & 15)) * 16);
    int a_ld[2][2];                                    // [K half][16-byte part]
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int s = 0; s < 2; ++s) a_ld[h][s] = lr * kRowA + (((8 * h + 4 * s + lq) ^ lr) * 16);

    f32x4 acc[NRF][NF];
#pragma unroll
    for (int i = 0; i < NRF; ++i)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x4v breg[NB][NF][2];
    uint2 bsreg[NB][NF];
    vec16 areg[APD][PASSES];
    uint2 sareg[APD];
    const int last = nch - 1;

    auto load_b = [&](i32x4v (&dst)[NF][2], uint2 (&ds)[NF], int c) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const unsigned char* p = Bg + boff[f] + static_cast<int64_t>(c) * (kChunk / 2);
            dst[f][0] = *reinterpret_cast<const i32x4v*>(p);
            dst[f][1] = *reinterpret_cast<const i32x4v*>(p + 64);
            ds[f] = *reinterpret_cast<const uint2*>(Sg + soff[f] + c * (kChunk / kBlk));
        }
    };
    auto load_a = [&](vec16 (&dst)[PASSES], uint2& ds, int c) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < PASSES; ++i) dst[i] = ld16(Abase + aoff[i] + static_cast<int64_t>(c) * kChunk);
        if (tid < BM) ds = *reinterpret_cast<const uint2*>(sa_src + c * (kChunk / kBlk));
    };
    auto store_a = [&](const vec16 (&src)[PASSES], uint2 ds, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < PASSES; ++i) st16(&s_a[buf][a_st + i * ROWS_PER_PASS * kRowA], src[i]);
        if (tid < BM) s_sa[buf][tid] = ds;
    };
    auto compute = [&](const i32x4v (&bv)[NF][2], const uint2 (&bs)[NF], int buf) __attribute__((always_inline)) {
        const unsigned char* src = s_a[buf];
        const unsigned char* ssa = reinterpret_cast<const unsigned char*>(s_sa[buf]);
        // this lane's weight-scale byte for each K half: byte lq (half 0) and 4 + lq (half 1)
        int sb[NF][2];
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            sb[f][0] = static_cast<int>(bs[f].x >> (8 * lq));
            sb[f][1] = static_cast<int>(bs[f].y >> (8 * lq));
        }
#pragma unroll
        for (int i = 0; i < NRF; ++i) {
            if (i == 0 || i < nrf) {
                const unsigned char* ri = src + i * 16 * kRowA;
                const int arow = (i * 16 + lr) * 8;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const vec16 lo = ld16(ri + a_ld[h][0]);
                    const vec16 hi = ld16(ri + a_ld[h][1]);
                    const i32x8 av = {static_cast<int>(lo.w[0]), static_cast<int>(lo.w[1]), static_cast<int>(lo.w[2]),
                                      static_cast<int>(lo.w[3]), static_cast<int>(hi.w[0]), static_cast<int>(hi.w[1]),
                                      static_cast<int>(hi.w[2]), static_cast<int>(hi.w[3])};
                    const int sa = ssa[arow + 4 * h + lq];
#pragma unroll
                    for (int f = 0; f < NF; ++f) {
                        const i32x4v b4 = bv[f][h];
                        const i32x8 b8 = {b4[0], b4[1], b4[2], b4[3], 0, 0, 0, 0};
                        acc[i][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b8, acc[i][f], 0, 4, 0, sa, 0,
                                                                                    sb[f][h]);
                    }
                }
            }
        }
    };

    // ---- main loop: loads of chunk c + APD (A) and c + PD (B) in flight
    // while chunk c is multiplied; the A tile is double-buffered in LDS ------
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
    if (c < nch) step(std::integral_constant<int, 0>{}, c);

    // ---- epilogue ------------------------------------------------------------
    const int64_t crow0 = shared ? m0 : static_cast<int64_t>(row0) + m0;
    if constexpr (EPI == Epi::SWIGLU) {
        // h = silu(g) * u in fp32, then MX e4m3: one shared exponent per
        // (row, 32 h columns). With 4 wavefronts a wavefront's 32 columns are
        // one block; with 8, two wavefronts share a block through LDS.
        float h[NRF][NF / 2][4];
        int X[NRF][4];
#pragma unroll
        for (int i = 0; i < NRF; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float m = 0.0f;
#pragma unroll
                for (int f = 0; f < NF / 2; ++f) {
                    const float gv = acc[i][f][v], uv = acc[i][f + NF / 2][v];
                    h[i][f][v] = gv / (1.0f + __expf(-gv)) * uv;
                    m = fmaxf(m, fabsf(h[i][f][v]));
                }
#pragma unroll
                for (int s = 1; s < 16; s <<= 1) m = fmaxf(m, __shfl_xor(m, s, 16));
                if constexpr (WPB > 1) {
                    if (lr == 0) s_amax[wave][i * 16 + lq * 4 + v] = m;
                } else {
                    X[i][v] = mx_exponent(m);
                }
            }
        if constexpr (WPB > 1) {
            __syncthreads();
            const int w0 = wave - wave % WPB;
#pragma unroll
            for (int i = 0; i < NRF; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = i * 16 + lq * 4 + v;
                    float m = s_amax[w0][r];
#pragma unroll
                    for (int w = 1; w < WPB; ++w) m = fmaxf(m, s_amax[w0 + w][r]);
                    X[i][v] = mx_exponent(m);
                }
        }
        uint8_t* Cq = static_cast<uint8_t*>(shared ? a.C_shared : a.C);
        uint8_t* Cs = static_cast<uint8_t*>(shared ? a.C_scale_shared : a.C_scale);
        const int nsb = a.N / kBlk;
        const int col0 = nt * 128 + wave * CPW;
#pragma unroll
        for (int i = 0; i < NRF; ++i) {
            if (i < nrf) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = i * 16 + lq * 4 + v;
                    if (r < rows) {
                        const float inv = mx_inv_scale(X[i][v]);
#pragma unroll
                        for (int f = 0; f < NF / 2; ++f) {
                            const uint32_t code = cvt2_e4m3_sat(h[i][f][v] * inv, 0.0f) & 0xffu;
                            Cq[(crow0 + r) * a.ldc + col0 + 16 * f + lr] = static_cast<uint8_t>(code);
                        }
                        if (lr == 0 && wave % WPB == 0)
                            Cs[(crow0 + r) * nsb + col0 / kBlk] = static_cast<uint8_t>(X[i][v] + 127);
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

template <Epi EPI>
hipError_t launch_mx_bm(const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(p.grid));
    if (p.nw == 4 && p.bm == 32) {
        hipLaunchKernelGGL((gemm_mx_kernel<EPI, 32, 4>), grid, dim3(256), 0, s, a, p.n_tiles);
    } else if (p.nw == 8 && p.bm == 64) {
        hipLaunchKernelGGL((gemm_mx_kernel<EPI, 64, 8>), grid, dim3(512), 0, s, a, p.n_tiles);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_mx(const void* x_bf16, uint8_t* q, uint8_t* scale, int64_t rows, int cols, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_mx_kernel, dim3(static_cast<unsigned>(rows)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(x_bf16), q, scale, cols);
    return hipGetLastError();
}

GemmPlan plan_gemm_mx(Epi epi, int64_t rows_upper, int n_groups, int64_t expected_rows_per_group, int N) {
    GemmPlan p;
    p.nw = 4;
    p.smajor = 0;
    p.big = 0;
    p.ksplit = 1;
    // 32-row tiles on 4 wavefronts; 64-row tiles on 8 (two per SIMD), which
    // halves each wavefront's share of the weight fragments and accumulators.
    p.bm = expected_rows_per_group <= 32 ? 32 : 64;
    p.nw = p.bm == 32 ? 4 : 8;
    const int cols = epi == Epi::SWIGLU ? 128 : 256;
    p.n_tiles = (N + cols - 1) / cols;
    const int64_t m_tiles = rows_upper / p.bm + n_groups;
    p.grid = ((m_tiles * p.n_tiles + 7) / 8) * 8;
    return p;
}

hipError_t launch_gemm_mx(Epi epi, const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    if (p.grid == 0) return hipSuccess;
    if (a.K % kChunk != 0) return hipErrorInvalidValue;
    GemmArgs b = a;
    b.ksplit = 1;
    return epi == Epi::SWIGLU ? launch_mx_bm<Epi::SWIGLU>(b, p, s) : launch_mx_bm<Epi::PLAIN>(b, p, s);
}

}  // namespace moe
