// Shared-expert GEMM tiles small enough to run beside the routed experts'
// bandwidth-bound tiles on the same compute units.
//
// What it computes: the shared expert of the layer (Perplexity "Lower latency
// and higher throughput with multi-node DeepSeek deployment", section
// "Expert parallelism": one expert every token passes through), as the same
// SWIGLU / PLAIN grouped-GEMM steps as gemm.hip with a single group of T
// rows; NVIDIA "Optimizing DeepSeek R1 throughput on Blackwell", section
// "Multi-stream optimization": the shared expert runs concurrently with the
// routed experts.
//
// Why a separate kernel (MI355X): at decode shapes the routed tiles stream
// weights and leave the matrix cores mostly idle, but each of their
// workgroups holds 4 waves of about 374 registers (one per SIMD) and 48 KB of
// LDS. A 256 x 256 shared-expert workgroup needs a whole CU, so running the
// two concurrently only splits the CUs between them. These tiles fit in what
// a routed workgroup leaves free, so both run on every CU at once:
//  * 128 x 128 tiles, 4 waves as 2 x 2, each 64 rows x 64 weight rows as
//    32 x 32 fragments of v_mfma_f32_32x32x16_bf16; at most 128 registers
//    per wave;
//  * both operands go HBM/L2 -> LDS with global_load_lds_dwordx4 in whole
//    128-byte lines, K = 64 per stage, two stages (64 KB); the launch asks
//    for 80 KB so that a CU never holds two of these workgroups (which would
//    leave no room for a routed one) and always has 80 KB left;
//  * one persistent workgroup per CU walks its XCD's contiguous range of
//    tiles (n-tile major), so the workgroups of an XCD share weight panels in
//    its L2;
//  * the LDS swizzle, fragment layout and gate/up interleave are those of the
//    256 x 256 tiles (gemm_big.hip).
#include <algorithm>
#include <atomic>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kCBM = 128;                  // rows per tile
constexpr int kCBN = 128;                  // weight rows per tile
constexpr int kCKB = 64;                   // K per stage
constexpr int kCRowB = kCKB * 2;           // 128 LDS bytes per row per stage
constexpr int kCGran = kCRowB / 16;        // 8 granules per row
constexpr int kCStageB = (kCBM + kCBN) * kCRowB;   // 32 KB
constexpr int kCLdsUsed = 2 * kCStageB;            // 64 KB
constexpr int kCLdsAsk = 80 * 1024;
constexpr int kCThreads = 256;
constexpr int kCLoads = kCBM * kCGran / kCThreads;  // 4 direct loads per operand per stage per thread
constexpr int kCRowsPerLoad = 64 / kCGran;          // 8 rows per load instruction
static_assert(kCBM == kCBN, "the load loop assumes equal operand tiles");
static_assert(kCLdsAsk >= kCLdsUsed, "");

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int cswz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ bf16x8 cfrag(const unsigned char* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const vec16*>(p));
}

__device__ __forceinline__ void cload_lds16(const void* g, unsigned char* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

constexpr int cwaitcnt(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// Wait for this thread's direct loads and LDS reads, then a bare barrier.
__device__ __forceinline__ void csync() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(cwaitcnt(0, 0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// One group of T rows (the shared expert): x [T, K] and the weights
// [N_w, K] bf16 row-major. SWIGLU: weight rows 0..inter-1 gate, inter..2*inter-1
// up; C = h [T, inter] bf16. PLAIN: C [T, N] fp32 (out_f32) or bf16.
template <Epi EPI>
__global__ __launch_bounds__(kCThreads) __attribute__((amdgpu_waves_per_eu(4)))
void gemm_cores_kernel(GemmArgs a, int n_tiles, int m_tiles) {
    extern __shared__ __attribute__((aligned(16))) unsigned char s_ring[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int K = a.K;
    const int nkb = K / kCKB;
    const int total = m_tiles * n_tiles;
    const int per_xcd = (total + 7) >> 3;
    const int wg_per_xcd = static_cast<int>(gridDim.x >> 3);
    const int xcd = static_cast<int>(blockIdx.x & 7);
    const unsigned char* Ag = static_cast<const unsigned char*>(a.A_shared);
    const unsigned char* Bg = static_cast<const unsigned char*>(a.B_shared);
    const int lrow = lane / kCGran;

    // fragment reads: lane l reads row l % 32 of a 32-row block, granule
    // 2t + l / 32 of k-step t
    const int fr = lane & 31;
    int f_off[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) f_off[t] = fr * kCRowB + (((2 * t + (lane >> 5)) ^ cswz(fr)) * 16);
    const int a_base = wm * 64 * kCRowB;
    const int b_base = kCBM * kCRowB + wn * 64 * kCRowB;

    for (int slot = static_cast<int>(blockIdx.x >> 3); slot < per_xcd; slot += wg_per_xcd) {
        const int L = xcd * per_xcd + slot;
        if (L >= total) break;                              // uniform
        const int nt = L / m_tiles, mt = L - (L / m_tiles) * m_tiles;
        const int m0 = mt * kCBM;
        const int rows = min(kCBM, a.T - m0);

        uint32_t aoff[kCLoads], boff[kCLoads];
#pragma unroll
        for (int j = 0; j < kCLoads; ++j) {
            const int rs = (4 * j + wave) * kCRowsPerLoad + lrow;      // tile row this lane fills
            const int r = rs < rows ? rs : rows - 1;                   // past the end: a valid row, unused
            aoff[j] = static_cast<uint32_t>(m0 + r) * static_cast<uint32_t>(K * 2) + ((lane % kCGran) ^ cswz(rs)) * 16;
            const int n = rs;                                          // weight row slot of the tile
            int brow;
            if constexpr (EPI == Epi::SWIGLU) {
                // slots [64 wn, 64 wn + 64): 32 gate rows then the 32 up rows
                // of the same h columns
                int col = nt * 64 + (n / 64) * 32 + (n % 32);
                col = col < a.inter ? col : a.inter - 1;               // column tail: valid row, result dropped
                brow = (n & 32) ? a.inter + col : col;
            } else {
                brow = nt * kCBN + n;
                brow = brow < a.N ? brow : a.N - 1;
            }
            boff[j] = static_cast<uint32_t>(brow) * static_cast<uint32_t>(K * 2) + ((lane % kCGran) ^ cswz(n)) * 16;
        }
        auto issue = [&](int kb, int stage) __attribute__((always_inline)) {
            unsigned char* sa = s_ring + stage * kCStageB;
            unsigned char* sb = sa + kCBM * kCRowB;
            const uint32_t ko = static_cast<uint32_t>(kb) * kCRowB;
#pragma unroll
            for (int j = 0; j < kCLoads; ++j)
                cload_lds16(Ag + aoff[j] + ko, sa + (4 * j + wave) * kCRowsPerLoad * kCRowB);
#pragma unroll
            for (int j = 0; j < kCLoads; ++j)
                cload_lds16(Bg + boff[j] + ko, sb + (4 * j + wave) * kCRowsPerLoad * kCRowB);
        };

        const int nrb = (rows + 31) >> 5;                  // 32-row blocks with data
        const int nbw = min(max(nrb - wm * 2, 0), 2);      // of this wave's 2 (uniform)
        f32x16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

        // two LDS stages: at the top of iteration kb stage kb has landed
        // everywhere and stage kb - 1's slot is free; the loads of stage
        // kb + 1 then run while stage kb is multiplied
        issue(0, 0);
        for (int kb = 0; kb < nkb; ++kb) {
            csync();
            if (kb + 1 < nkb) issue(kb + 1, (kb + 1) & 1);
            const unsigned char* st = s_ring + (kb & 1) * kCStageB;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                bf16x8 af[2], bfr[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) af[i] = cfrag(st + a_base + i * 32 * kCRowB + f_off[t]);
#pragma unroll
                for (int j = 0; j < 2; ++j) bfr[j] = cfrag(st + b_base + j * 32 * kCRowB + f_off[t]);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    if (i < nbw) {
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
                    }
                }
            }
        }
        // every thread's loads have landed and its LDS reads are done before
        // the next tile's first loads overwrite the stages
        csync();

        // epilogue: lane l holds column l % 32 and rows 8 (e / 4) + 4 (l / 32)
        // + e % 4 of each 32 x 32 fragment
        const int lc = lane & 31, lh = lane >> 5;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (i < nbw) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int r = wm * 64 + i * 32 + (e >> 2) * 8 + lh * 4 + (e & 3);
                    if (r < rows) {
                        const int64_t rb = static_cast<int64_t>(m0 + r) * a.ldc;
                        if constexpr (EPI == Epi::SWIGLU) {
                            const int col = nt * 64 + wn * 32 + lc;
                            if (col < a.N) {
                                const float g = acc[i][0][e], u = acc[i][1][e];
                                reinterpret_cast<uint16_t*>(a.C_shared)[rb + col] =
                                    f32_to_bf16_bits(silu_mul(g, u));
                            }
                        } else {
#pragma unroll
                            for (int j = 0; j < 2; ++j) {
                                const int col = nt * kCBN + wn * 64 + j * 32 + lc;
                                if (col < a.N) {
                                    if (a.out_f32)
                                        reinterpret_cast<float*>(a.C_shared)[rb + col] = acc[i][j][e];
                                    else
                                        reinterpret_cast<uint16_t*>(a.C_shared)[rb + col] = f32_to_bf16_bits(acc[i][j][e]);
                                }
                            }
                        }
                    }
                }
            }
        }
    }
}

template <Epi EPI>
hipError_t launch_cores_epi(const GemmArgs& a, const GemmPlan& p, int m_tiles, hipStream_t s) {
    static std::atomic<int> lds_set[kMaxDevices];
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&gemm_cores_kernel<EPI>), kCLdsAsk, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_cores_kernel<EPI>), dim3(static_cast<unsigned>(p.grid)), dim3(kCThreads), kCLdsAsk, s, a,
                       p.n_tiles, m_tiles);
    return hipGetLastError();
}

}  // namespace

GemmPlan plan_gemm_cores(Epi epi, int64_t T, int N, int cus) {
    GemmPlan p;
    p.bm = kCBM;
    p.nw = 4;
    p.smajor = 0;
    p.ksplit = 1;
    p.big = 0;
    p.n_tiles = epi == Epi::SWIGLU ? (N + 63) / 64 : (N + kCBN - 1) / kCBN;
    const int64_t tiles = (T + kCBM - 1) / kCBM * p.n_tiles;
    // one persistent workgroup per CU, a multiple of 8 (the XCD dealing)
    int64_t grid = std::max<int64_t>(8, cus / 8 * 8);
    grid = std::min<int64_t>(grid, (tiles + 7) / 8 * 8);
    p.grid = grid;
    return p;
}

hipError_t launch_gemm_cores(Epi epi, const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    if (p.grid == 0 || a.T == 0) return hipSuccess;
    if (a.K % kCKB != 0 || a.n_local != 0 || !a.has_shared) return hipErrorInvalidValue;
    // byte offsets into x and the weights are 32-bit
    const int64_t wrows = epi == Epi::SWIGLU ? 2 * static_cast<int64_t>(a.inter) : a.N;
    if (static_cast<int64_t>(std::max<int64_t>(a.T, wrows)) * a.K * 2 >= (int64_t{1} << 32)) return hipErrorInvalidValue;
    const int m_tiles = (a.T + kCBM - 1) / kCBM;
    return epi == Epi::SWIGLU ? launch_cores_epi<Epi::SWIGLU>(a, p, m_tiles, s)
                              : launch_cores_epi<Epi::PLAIN>(a, p, m_tiles, s);
}

}  // namespace moe
