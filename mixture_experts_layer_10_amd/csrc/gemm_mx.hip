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

// Workgroup barrier of the LDS double buffer: waits for this wavefront's LDS
// accesses (lgkmcnt 0) but not for its global loads (vmcnt left at its
// maximum), so the weight and activation loads of the chunks ahead stay in
// flight across it; __syncthreads would drain them every chunk.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);                 // vmcnt 63, expcnt 7, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

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
// columns). A chunk is CK elements of K: KH = CK / 128 MFMA steps, CK / 2
// bytes of each weight row. Weights go straight from HBM into VGPRs PD chunks
// ahead of use; the activation tile goes HBM/L2 -> VGPRs one chunk ahead and
// VGPRs -> LDS (double-buffered) at the end of the chunk before its use. The
// weight scales of the tile's 256 rows (K/32 bytes each) are read once, at
// the start, into LDS (dynamic shared memory, mx_scale_lds_bytes): read a few
// bytes per row per chunk from global memory instead, their cache lines are
// evicted by the streaming weights between chunks and fetched several times.
template <int N>
struct Bytes {                                          // N scale bytes held as N / 4 dwords
    uint32_t w[N / 4];
};
template <int N>
__device__ __forceinline__ Bytes<N> ld_bytes(const unsigned char* p) {
    Bytes<N> b;
    if constexpr (N == 16) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        b.w[0] = v.x; b.w[1] = v.y; b.w[2] = v.z; b.w[3] = v.w;
    } else {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        b.w[0] = v.x; b.w[1] = v.y;
    }
    return b;
}

// Row stride of the staged weight scales: K/32 bytes plus 8, so that the 16
// rows of a fragment fall in different LDS banks.
__host__ __device__ constexpr int mx_scale_stride(int K) { return K / kBlk + 8; }
__host__ __device__ constexpr int mx_scale_lds_bytes(int K) { return 256 * mx_scale_stride(K); }

template <Epi EPI, int BM, int NW, int CK, int PD, int OCC>
__global__ __launch_bounds__(NW * 64, OCC) void gemm_mx_kernel(GemmArgs a, int n_tiles) {
    constexpr int NT = NW * 64;
    constexpr int NF = 16 / NW;                        // 16-row fragments per wavefront
    constexpr int NRF = BM / 16;
    constexpr int KH = CK / 128;                       // MFMA K-steps per chunk
    constexpr int ROWB = CK;                           // LDS bytes per A row per chunk (e4m3)
    constexpr int ROWG = CK / 16;                      // 16-byte granules per A row per chunk
    constexpr int SB = CK / kBlk;                      // scale bytes per row per chunk
    constexpr int ROWS_PER_PASS = NT / ROWG;
    constexpr int PASSES = BM / ROWS_PER_PASS;
    constexpr int NB = PD + 1;                         // weight register buffers
    constexpr int U = NB;                              // steps per unrolled body: every buffer index static
    static_assert(BM % ROWS_PER_PASS == 0, "tile rows");
    static_assert(BM <= NT, "one activation-scale loader per tile row");
    static_assert(KH == 2 || KH == 4, "chunk of 256 or 512");

    __shared__ __attribute__((aligned(16))) unsigned char s_a[2][BM * ROWB];
    __shared__ __attribute__((aligned(16))) unsigned char s_sa[2][BM * SB];
    constexpr int CPW = 16 * (NF / 2);                              // SWIGLU: h columns per wavefront
    constexpr int WPB = CPW >= kBlk ? 1 : kBlk / CPW;               // wavefronts per 32-column block
    __shared__ float s_amax[WPB > 1 ? NW : 1][WPB > 1 ? BM : 1];
    extern __shared__ __attribute__((aligned(16))) unsigned char s_bs[];   // [256][kbp] weight scales

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
    const int nch = K / CK;
    const int kb = K / kBlk;                           // scale bytes per row

    // ---- weights: packed E2M1 rows (K/2 bytes) and E8M0 scales (K/32 bytes).
    // Bases are workgroup-uniform and offsets 32-bit, so the loads take the
    // scalar-base form and no 64-bit address per load sits in VGPRs.
    const int nb_rows = EPI == Epi::SWIGLU ? 2 * a.inter : a.N;
    const unsigned char* Bg = shared ? static_cast<const unsigned char*>(a.B_shared)
                                     : static_cast<const unsigned char*>(a.B) + static_cast<int64_t>(g) * a.b_stride;
    const unsigned char* Sg = shared ? static_cast<const unsigned char*>(a.B_scale_shared)
                                     : static_cast<const unsigned char*>(a.B_scale) +
                                           static_cast<int64_t>(g) * nb_rows * kb;
    const int kbp = mx_scale_stride(K);
    uint32_t boff[NF];
    int sb_ld[NF];                                     // LDS offset of this lane's row of weight scales
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
        const int trow = EPI == Epi::SWIGLU ? (f < NF / 2 ? wave * (128 / NW) + 16 * f + lr
                                                           : 128 + wave * (128 / NW) + 16 * (f - NF / 2) + lr)
                                            : wave * (256 / NW) + 16 * f + lr;
        sb_ld[f] = trow * kbp + lq;
    }
    // Stage the tile's weight scales: tile row j is weight row
    // (SWIGLU) nt*128 + j (gate) or inter + nt*128 + j - 128 (up), or
    // (PLAIN) nt*256 + j clamped to N - 1; 8 bytes per load, consecutive
    // threads on consecutive bytes of a row. Called once, after the first
    // chunk's loads are issued and before the first barrier. Loads go out in
    // batches of kScaleBatch before their stores (a load past the end reads
    // the last element again and is not stored), so a thread waits once per
    // batch instead of once per load.
    auto stage_scales = [&]() __attribute__((always_inline)) {
        constexpr int kScaleBatch = 7;
        const int vpr = kb / 8;
        const int total = 256 * vpr;
        auto src = [&](int v) -> uint32_t {
            v = v < total ? v : total - 1;
            const int j = v / vpr, q = v - j * vpr;
            int wrow;
            if constexpr (EPI == Epi::SWIGLU) wrow = j < 128 ? nt * 128 + j : a.inter + nt * 128 + (j - 128);
            else wrow = min(nt * 256 + j, a.N - 1);
            return static_cast<uint32_t>(wrow) * kb + q * 8;
        };
        for (int v0 = tid; v0 < total; v0 += kScaleBatch * NT) {
            uint2 val[kScaleBatch];
#pragma unroll
            for (int s = 0; s < kScaleBatch; ++s) val[s] = *reinterpret_cast<const uint2*>(Sg + src(v0 + s * NT));
#pragma unroll
            for (int s = 0; s < kScaleBatch; ++s) {
                const int v = v0 + s * NT;
                if (v < total) {
                    const int j = v / vpr, q = v - j * vpr;
                    *reinterpret_cast<uint2*>(s_bs + j * kbp + q * 8) = val[s];
                }
            }
        }
    };

    // ---- activations: gathered e4m3 rows and their scale bytes ------------
    const int aj = tid % ROWG, ar = tid / ROWG;
    const unsigned char* Ag = static_cast<const unsigned char*>(shared ? a.A_shared : a.A);
    const unsigned char* Asg = static_cast<const unsigned char*>(shared ? a.A_scale_shared : a.A_scale);
    auto src_row = [&](int r) -> uint32_t {
        r = r < rows ? r : rows - 1;
        if (shared) return m0 + r;
        if (a.gather) return static_cast<uint32_t>(a.perm[row0 + m0 + r] / a.topk);
        return row0 + m0 + r;
    };
    uint32_t aoff[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) aoff[i] = src_row(ar + i * ROWS_PER_PASS) * static_cast<uint32_t>(K) + aj * 16;
    const uint32_t sao = tid < BM ? src_row(tid) * static_cast<uint32_t>(kb) : 0u;
    // LDS: row r's granule j sits at j ^ (r & 15): the 16 rows of a fragment
    // read 16 different granule slots, so the 64 lanes' reads spread over all banks.
    const int a_st = ar * ROWB + ((aj ^ (ar & 15)) * 16);
    const int a_ld = lr * ROWB;

    f32x4 acc[NRF][NF];
#pragma unroll
    for (int i = 0; i < NRF; ++i)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x4v breg[NB][NF][KH];
    vec16 areg[PASSES];
    Bytes<SB> sareg;
    const int last = nch - 1;

    auto load_b = [&](i32x4v (&dst)[NF][KH], int c) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const uint32_t o = boff[f] + static_cast<uint32_t>(c) * (CK / 2);
#pragma unroll
            for (int h = 0; h < KH; ++h) dst[f][h] = *reinterpret_cast<const i32x4v*>(Bg + (o + h * 64));
        }
    };
    auto load_a = [&](int c) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < PASSES; ++i) areg[i] = ld16(Ag + (aoff[i] + static_cast<uint32_t>(c) * CK));
        if (tid < BM) sareg = ld_bytes<SB>(Asg + (sao + static_cast<uint32_t>(c) * SB));
    };
    auto store_a = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < PASSES; ++i) st16(&s_a[buf][a_st + i * ROWS_PER_PASS * ROWB], areg[i]);
        if (tid < BM) {
            if constexpr (SB == 16)
                *reinterpret_cast<uint4*>(&s_sa[buf][tid * SB]) = make_uint4(sareg.w[0], sareg.w[1], sareg.w[2], sareg.w[3]);
            else
                *reinterpret_cast<uint2*>(&s_sa[buf][tid * SB]) = make_uint2(sareg.w[0], sareg.w[1]);
        }
    };
    auto compute = [&](const i32x4v (&bv)[NF][KH], int c, int buf) __attribute__((always_inline)) {
        const unsigned char* src = s_a[buf];
        const unsigned char* ssa = s_sa[buf];
        const unsigned char* sbs = s_bs + c * SB;
        int sb[NF][KH];                                // weight scale of K block 4h + lq of this lane's row
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int h = 0; h < KH; ++h) sb[f][h] = sbs[sb_ld[f] + 4 * h];
#pragma unroll
        for (int i = 0; i < NRF; ++i) {
            if (i == 0 || i < nrf) {
                const unsigned char* ri = src + i * 16 * ROWB + a_ld;
                const int arow = (i * 16 + lr) * SB;
#pragma unroll
                for (int h = 0; h < KH; ++h) {
                    // this lane's e4m3 bytes: K = 16 lq .. and 64 + 16 lq .. of step h
                    const vec16 lo = ld16(ri + (((8 * h + lq) ^ lr) * 16));
                    const vec16 hi = ld16(ri + (((8 * h + 4 + lq) ^ lr) * 16));
                    const i32x8 av = {static_cast<int>(lo.w[0]), static_cast<int>(lo.w[1]), static_cast<int>(lo.w[2]),
                                      static_cast<int>(lo.w[3]), static_cast<int>(hi.w[0]), static_cast<int>(hi.w[1]),
                                      static_cast<int>(hi.w[2]), static_cast<int>(hi.w[3])};
                    const int sa = ssa[arow + 4 * h + lq];           // scale of K block 4h + lq
#pragma unroll
                    for (int f = 0; f < NF; ++f) {
                        const i32x4v b4 = bv[f][h];
                        const i32x8 b8 = {b4[0], b4[1], b4[2], b4[3], 0, 0, 0, 0};
                        acc[i][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            av, b8, acc[i][f], 0, 4, 0, sa, 0, sb[f][h]);
                    }
                }
            }
        }
    };

    // ---- main loop. Per chunk c: the activations of c + 1 are loaded first
    // and the weights of c + PD after them, so that waiting for the former
    // (to stage them into LDS at the end of the chunk) never waits for the
    // weights just issued; chunk c is multiplied in between. ----------------
    auto step = [&](auto uc, int c) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        load_a(min(c + 1, last));
        load_b(breg[(u + PD) % NB], min(c + PD, last));
        compute(breg[u % NB], c, c & 1);
        store_a((c + 1) & 1);
        lds_barrier();
    };
    if (nch > 0) {
        load_a(0);
#pragma unroll
        for (int p = 0; p < PD; ++p) load_b(breg[p], min(p, last));
        stage_scales();
        store_a(0);
        lds_barrier();
    }
    int c = 0;
    for (; c + U <= nch; c += U) {
        [&]<int... I>(std::integer_sequence<int, I...>) {
            (step(std::integral_constant<int, I>{}, c + I), ...);
        }(std::make_integer_sequence<int, U>{});
    }
    [&]<int... I>(std::integer_sequence<int, I...>) {           // at most U - 1 steps remain
        ((c + I < nch ? step(std::integral_constant<int, I>{}, c + I) : void()), ...);
    }(std::make_integer_sequence<int, U - 1>{});

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
                    h[i][f][v] = silu_mul(gv, uv);
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

template <Epi EPI, int BM, int NW, int CK, int PD, int OCC>
hipError_t launch_mx_one(const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    auto* kern = &gemm_mx_kernel<EPI, BM, NW, CK, PD, OCC>;
    const int dyn = mx_scale_lds_bytes(a.K);
    static std::atomic<int> lds_set[kMaxDevices];
    const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), dyn, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(p.grid)), dim3(NW * 64), static_cast<size_t>(dyn), s, a,
                       p.n_tiles);
    return hipGetLastError();
}

template <Epi EPI>
hipError_t launch_mx_bm(const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    if (p.nw == 4 && p.bm == 32) return launch_mx_one<EPI, 32, 4, 256, 1, 2>(a, p, s);
    if (p.nw == 8 && p.bm == 64) return launch_mx_one<EPI, 64, 8, 256, 1, 2>(a, p, s);
    return hipErrorInvalidValue;
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
    // 32-row tiles on 4 wavefronts, 64-row tiles on 8 (two per SIMD, each
    // holding half the weight fragments); one chunk of weights in flight
    // beyond the one being multiplied.
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
    if (a.K % 256 != 0) return hipErrorInvalidValue;
    GemmArgs b = a;
    b.ksplit = 1;
    return epi == Epi::SWIGLU ? launch_mx_bm<Epi::SWIGLU>(b, p, s) : launch_mx_bm<Epi::PLAIN>(b, p, s);
}

}  // namespace moe
