// K5 / K6 at compute-bound shapes (bf16): grouped GEMM with 256 x 256 tiles
// staged through LDS (double-buffered) by direct global -> LDS loads.
//
// What it computes is that of gemm.hip (Perplexity "Lower latency and higher
// throughput with multi-node DeepSeek deployment", section "Roofline >
// GroupGEMM": per group, rows x weight^T; SWIGLU epilogue h = silu(gate) * up,
// infra guide "Data parallelism and expert parallelism", section 2.1). This
// variant is for groups of hundreds of rows (prefill), where the product is
// bound by matrix throughput rather than by streaming the weights once:
//
//  * a workgroup computes 256 rows x 256 weight rows; its NW wavefronts
//    (8 by default, two per SIMD; 4 also built) form 2 x NW/2 and each
//    computes four 32-row blocks x 512/NW weight rows as 32 x 32 fragments
//    of v_mfma_f32_32x32x16_bf16;
//  * both operands go HBM/L2 -> LDS with buffer_load_dwordx4 ... lds (no
//    VGPR staging; 32-bit row offsets against a buffer descriptor, the stage
//    offset in a scalar), K = 64 per stage: each row's 128 bytes are one whole cache
//    line, so a load instruction touches 8 lines (half-line loads, 16 rows of
//    64 bytes, ran about a third slower); two stages (128 KB);
//  * one barrier per stage, placed mid-stage: the MFMAs of a stage's last two
//    k-steps run while the next stage's first fragments are read and the
//    stage after next is loaded;
//  * 16-byte granule q of LDS row r sits at q ^ ((r >> 1) & 7), which makes
//    the fragment reads (32 rows x one granule per lane half) free of bank
//    conflicts (measured with the bank-conflict counter); the direct loads
//    fill 8 rows per instruction, lane l taking the granule that the swizzle
//    puts at its position;
//  * SwiGLU tiles interleave gate and up rows so that each wavefront holds
//    matching gate and up columns: h = silu(g) * u is formed in registers;
//  * a group's rows are split evenly over its m-tiles, and 32-row blocks past
//    a tile's real row count are neither read nor multiplied; in such a short
//    tile the two wavefront rows take alternate blocks, so its busier row
//    does ceil(blocks / 2) blocks of work rather than min(blocks, 4);
//  * the K loop is instantiated for each count of a wavefront's blocks with
//    data (0..4), so it holds no branch, and scheduling groups make its
//    MFMAs alternate with the fragment reads.
#include <utility>

#include "gemm_tile.h"

namespace moe {
namespace {

constexpr int kBM = 256;                  // rows per tile
constexpr int kBN = 256;                  // weight rows per tile
constexpr int kKB = 64;                   // K per stage
constexpr int kRowB = kKB * 2;            // 128 LDS bytes per row per stage: whole cache lines
constexpr int kGran = kRowB / 16;         // 16-byte granules per row
constexpr int kStages = 2;
constexpr int kStageB = (kBM + kBN) * kRowB;   // 64 KB

// LDS swizzle: granule q of row r sits at q ^ ((r >> 1) & 7).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 lds_frag(const unsigned char* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const vec16*>(p));
}


// s_waitcnt immediate (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]).
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// NW wavefronts as 2 (rows) x NW/2 (columns); each computes four 32-row
// blocks x WB = 512 / NW weight rows. With NW = 8 two wavefronts share each SIMD, so
// one issues MFMAs while the other waits at a barrier or on LDS.
template <Epi EPI, int NW>
__global__ __launch_bounds__(NW * 64, 1) void gemm_big_kernel(GemmArgs a, int n_tiles) {
    constexpr int NT = NW * 64;
    constexpr int WB = 2 * kBN / NW;                 // weight rows per wavefront
    constexpr int NJ = WB / 32;                      // 32-column fragments per wavefront
    constexpr int kLoads = kBM * kGran / NT;         // direct loads per thread per operand per stage
    constexpr int kRowsPerLoad = 64 / kGran;         // rows one direct load fills (1 KB)
    extern __shared__ __attribute__((aligned(16))) unsigned char s_ring[];   // kStages x kStageB

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);      // wave-uniform (scalar branches)
    const int wm = wave & 1, wn = wave >> 1;

    Tile tl;
    if (!find_tile(a, n_tiles, kBM, tl, /*balanced=*/true)) return;
    const int g = tl.g, nt = tl.nt;
    const bool shared = tl.shared;
    const int row0 = tl.row0, m0 = tl.m0, rows = tl.rows;
    const int K = a.K;                                             // row length of both operands
    // With a K split (dense PLAIN fp32 only, checked at launch) the tile
    // multiplies K slice tl.ks and writes its partial sums.
    const int KS = a.ksplit;
    const int k_len = K / KS;
    const int64_t k_off = static_cast<int64_t>(tl.ks) * k_len * 2;  // bytes into each row
    const int nkb = k_len / kKB;
    const int last = nkb - 1;

    // ---- direct-load sources: instruction j of wavefront w fills rows
    // (NW j + w) * 8 + lane / 8 of the stage, granule slot lane % 8, and
    // loads the granule the swizzle places there --------------------------
    const int lrow = lane / kGran;                                 // row within the instruction's rows
    auto slot_granule = [&](int row) { return (lane % kGran) ^ swz(row); };
    const unsigned char* Ag = static_cast<const unsigned char*>(shared ? a.A_shared : a.A) + k_off;
    uint32_t aoff[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const int rs = (NW * j + wave) * kRowsPerLoad + lrow;
        const int r = rs < rows ? rs : rows - 1;                    // rows past the end: a valid row, unused
        uint32_t src;
        if (shared) src = m0 + r;
        else if (a.gather) src = static_cast<uint32_t>(a.perm[row0 + m0 + r] / a.topk);
        else src = row0 + m0 + r;
        aoff[j] = src * static_cast<uint32_t>(K * 2) + slot_granule(rs) * 16;
    }
    const unsigned char* Bg = (shared ? static_cast<const unsigned char*>(a.B_shared)
                               : static_cast<const unsigned char*>(a.B) + static_cast<int64_t>(g) * a.b_stride * 2) +
                              k_off;
    uint32_t boff[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const int n = (NW * j + wave) * kRowsPerLoad + lrow;       // weight row slot of the tile
        int brow;
        if constexpr (EPI == Epi::SWIGLU) {
            // slots [WB wn, WB wn + WB): WB/2 gate rows then the WB/2 up rows
            // of the same h columns
            int col = nt * 128 + (n / WB) * (WB / 2) + (n % (WB / 2));
            col = col < a.inter ? col : a.inter - 1;                // column tail: valid row, result dropped
            brow = (n & (WB / 2)) ? a.inter + col : col;
        } else {
            brow = nt * kBN + n;
            brow = brow < a.N ? brow : a.N - 1;
        }
        boff[j] = static_cast<uint32_t>(brow) * static_cast<uint32_t>(K * 2) + slot_granule(n) * 16;
    }
    // Both operands through buffer descriptors (offsets below 4 GiB: the
    // operand size limit): a load sends 32-bit row offsets, and the stage
    // offset rides in a scalar.
    const __amdgpu_buffer_rsrc_t ares = byte_buffer(Ag, 0xFFFFFFFFu), bres = byte_buffer(Bg, 0xFFFFFFFFu);
    auto issue = [&](int kb, int stage) __attribute__((always_inline)) {
        unsigned char* sa = s_ring + stage * kStageB;
        unsigned char* sb = sa + kBM * kRowB;
        const int ko = kb * kRowB;
#pragma unroll
        for (int j = 0; j < kLoads; ++j) buf_load_lds16(ares, aoff[j], ko, sa + (NW * j + wave) * kRowsPerLoad * kRowB);
#pragma unroll
        for (int j = 0; j < kLoads; ++j) buf_load_lds16(bres, boff[j], ko, sb + (NW * j + wave) * kRowsPerLoad * kRowB);
    };

    // ---- fragment reads: lane l reads row (l % 32) of a 32-row block,
    // granule 2t + l / 32 of k-step t ------------------------------------------
    constexpr int KSTEPS = kKB / 16;
    const int fr = lane & 31;
    int f_off[KSTEPS];
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) f_off[t] = fr * kRowB + (((2 * t + (lane >> 5)) ^ swz(fr)) * 16);
    const int b_base = kBM * kRowB + wn * WB * kRowB;
    const int nrb = (rows + 31) >> 5;                               // 32-row blocks with data

    f32x16 acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};

    // Block i of wavefront row wm is the tile's 32-row block b0 + i * bs. A
    // full tile gives each row four consecutive blocks; a tile cut short by
    // its group's row count alternates them (row wm takes blocks wm, wm + 2,
    // wm + 4, wm + 6), so both rows keep about equal work: the MFMAs of a
    // block with no rows are skipped, and a tile lasts as long as its busier
    // row. nbw = blocks of this wavefront that hold data (uniform: scalar
    // branches).
    const bool full = nrb == 8;
    const int b0 = full ? wm * 4 : wm, bs = full ? 1 : 2;
    const int nbw = full ? 4 : min(max((nrb - wm + 1) >> 1, 0), 4);
    int a_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a_off[i] = (b0 + i * bs) * 32 * kRowB;
    // Wait for this thread's LDS fills and LDS reads, then a bare barrier
    // (no fence: the fills are waited for explicitly). The empty asm
    // statements keep the compiler from moving memory accesses across it,
    // the scheduling barriers keep MFMAs on their side of it.
    auto sync = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- pipeline (two LDS slots) -------------------------------------------
    // Iteration kb: MFMAs of k-steps 0-1 of stage kb while its k-steps 2-3 are
    // read; then one barrier (stage kb+1 has landed everywhere, no one reads
    // stage kb's slot any more); then the loads of stage kb+2 into that slot
    // and the reads of stage kb+1's first k-steps are issued while k-steps 2-3
    // of stage kb run. Every wait is for all of a thread's outstanding loads,
    // so the last two iterations simply issue none (measured: +0.4% on the
    // prefill layer against reloading the last stage).
    //
    // The loop is instantiated for each count NBW of this wavefront's blocks
    // with data (0..4; the two wavefront rows of a short tile can differ), so
    // it holds no branch, reads only those blocks' fragments, and scheduling
    // groups fix the order of each half: MFMAs alternate with the fragment
    // reads (and after the barrier with the next stage's loads), which land
    // while later MFMAs run. Every variant runs the same barriers.
    auto kloop = [&](auto nbw_c) __attribute__((always_inline)) {
        constexpr int NBW = decltype(nbw_c)::value;
        // Fragments of k-steps 0..3 of a stage (4 x (NBW A + NJ B) registers).
        bf16x8 af[KSTEPS][NBW > 0 ? NBW : 1], bfr[KSTEPS][NJ];
        auto read = [&](int slot, int t) __attribute__((always_inline)) {
            const unsigned char* st = s_ring + slot * kStageB;
#pragma unroll
            for (int i = 0; i < NBW; ++i) af[t][i] = lds_frag(st + a_off[i] + f_off[t]);
#pragma unroll
            for (int j = 0; j < NJ; ++j) bfr[t][j] = lds_frag(st + b_base + j * 32 * kRowB + f_off[t]);
        };
        auto mfma = [&](int t) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < NBW; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t][i], bfr[t][j], acc[i][j], 0, 0, 0);
        };
        // scheduling groups (mask 0x008 MFMA, 0x100 LDS read, 0x010 VMEM):
        // M MFMAs, the first of them each followed by one of D reads, the
        // rest by one of V loads; whatever is left over goes last
        auto groups = [&](auto m_c, auto d_c, auto v_c) __attribute__((always_inline)) {
            constexpr int M = decltype(m_c)::value, D = decltype(d_c)::value, V = decltype(v_c)::value;
#pragma unroll
            for (int q = 0; q < M; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (q < D) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                else if (q - D < V) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
            }
            if constexpr (D > M) __builtin_amdgcn_sched_group_barrier(0x100, D - M, 0);
            if constexpr (V > 0 && D + V > M) __builtin_amdgcn_sched_group_barrier(0x010, D >= M ? V : D + V - M, 0);
        };
        constexpr int kRd = NBW + NJ;                          // fragment reads per k-step
        constexpr int kMf = NBW * NJ;                          // MFMAs per k-step
        issue(0, 0);
        sync();
        issue(min(1, last), 1);
        read(0, 0);
        read(0, 1);
        for (int kb = 0; kb < nkb; ++kb) {
            const int s = kb & 1;
            read(s, 2);
            mfma(0);
            read(s, 3);
            mfma(1);
            groups(std::integral_constant<int, 2 * kMf>{}, std::integral_constant<int, 2 * kRd>{},
                   std::integral_constant<int, 0>{});
            sync();
            if (kb + 2 <= last) issue(kb + 2, s);                // uniform
            read(s ^ 1, 0);
            read(s ^ 1, 1);
            // raised issue priority for the MFMAs that overlap the next
            // stage's loads and fragment reads: +0.8% at the prefill shape
            // (raising it for every k-step's MFMAs, or for the loads
            // instead, measured slower)
            __builtin_amdgcn_s_setprio(1);
            mfma(2);
            mfma(3);
            groups(std::integral_constant<int, 2 * kMf>{}, std::integral_constant<int, 2 * kRd>{},
                   std::integral_constant<int, 0>{});
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
        }
    };
    switch (nbw) {
        case 0: kloop(std::integral_constant<int, 0>{}); break;
        case 1: kloop(std::integral_constant<int, 1>{}); break;
        case 2: kloop(std::integral_constant<int, 2>{}); break;
        case 3: kloop(std::integral_constant<int, 3>{}); break;
        default: kloop(std::integral_constant<int, 4>{}); break;
    }
    // With a single stage the prologue's second (clamped) load may still be
    // landing: no direct-load write may outlive the workgroup's LDS.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

    // ---- epilogue: lane l holds column l % 32 and rows 8 (e / 4) + 4 (l / 32)
    // + e % 4 of each 32 x 32 fragment -----------------------------------------
    const int64_t crow0 = shared ? m0 : static_cast<int64_t>(row0) + m0;
    unsigned char* Cb = KS > 1 ? reinterpret_cast<unsigned char*>(a.partial + static_cast<int64_t>(tl.ks) * a.T * a.ldc)
                               : static_cast<unsigned char*>(shared ? a.C_shared : a.C);
    const int lc = lane & 31, lh = lane >> 5;
    // Outputs are staged in the (now idle) LDS ring as a row-major tile, then
    // written as whole 16-byte pieces of rows: a lane's own fragment values
    // are one column each, and storing them directly takes 2- or 4-byte
    // stores scattered over 16 rows per instruction (measured at the prefill
    // shape: the down GEMM's stores then cost about 13% of its time). A pass
    // covers the whole tile for bf16 outputs (at most 128 KB) and half of its
    // columns for fp32 outputs (two passes of 128 KB each).
    constexpr int TC = EPI == Epi::SWIGLU ? 128 : kBN;              // output columns of the tile
    auto epilogue = [&](auto f32_out) __attribute__((always_inline)) {
        constexpr bool F32 = decltype(f32_out)::value;
        constexpr int EB = F32 ? 4 : 2;                             // output bytes per element
        constexpr int PC = F32 ? TC / 2 : TC;                       // columns per pass
        constexpr int PRB = PC * EB;                                // LDS bytes per tile row in a pass
        constexpr int GPR = PRB / 16;                               // 16-byte pieces per row in a pass
        auto pass = [&](auto pass_c) __attribute__((always_inline)) {
            constexpr int P = decltype(pass_c)::value;
            __syncthreads();                   // fragment reads (or the previous pass's stores) are done
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (b0 + i * bs < nrb) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int r = (b0 + i * bs) * 32 + (e >> 2) * 8 + lh * 4 + (e & 3);
                        unsigned char* row = s_ring + r * PRB;
                        if constexpr (EPI == Epi::SWIGLU) {
#pragma unroll
                            for (int j = 0; j < NJ / 2; ++j)
                                reinterpret_cast<uint16_t*>(row)[wn * (WB / 2) + j * 32 + lc] =
                                    f32_to_bf16_bits(silu_mul(acc[i][j][e], acc[i][j + NJ / 2][e]));
                        } else {
#pragma unroll
                            for (int j = 0; j < NJ; ++j) {
                                const int col = wn * WB + j * 32 - P * PC;   // the fragment's first column in the pass
                                if (col >= 0 && col < PC) {                  // uniform: a fragment lies in one pass
                                    if constexpr (F32)
                                        reinterpret_cast<float*>(row)[col + lc] = acc[i][j][e];
                                    else
                                        reinterpret_cast<uint16_t*>(row)[col + lc] = f32_to_bf16_bits(acc[i][j][e]);
                                }
                            }
                        }
                    }
                }
            }
            __syncthreads();
            // N and ldc are multiples of 8 (checked at launch; layer sizes
            // are multiples of 128), so a 16-byte piece is either wholly
            // inside the output or wholly past its last column, and every
            // piece is aligned.
            const int c0 = nt * TC + P * PC;
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
    if constexpr (EPI == Epi::PLAIN) {
        if (a.out_f32) {
            epilogue(std::true_type{});
            return;
        }
    }
    epilogue(std::false_type{});
}

template <Epi EPI, int NW>
hipError_t launch_big_epi(const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    constexpr int lds = kStages * kStageB;
    static std::atomic<int> lds_set[kMaxDevices];
    const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&gemm_big_kernel<EPI, NW>), lds, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_big_kernel<EPI, NW>), dim3(static_cast<unsigned>(p.grid)), dim3(NW * 64), lds, s, a,
                       p.n_tiles);
    return hipGetLastError();
}

}  // namespace

// Plan of the 256 x 256 tile kernel: n_tiles column tiles (128 h columns for
// SWIGLU, 256 output columns for PLAIN), grid an upper bound on the tiles.
GemmPlan plan_gemm_big(Epi epi, int64_t rows_upper, int n_groups, int N) {
    GemmPlan p;
    p.bm = kBM;
    p.nw = 8;
    p.smajor = 0;
    p.ksplit = 1;
    p.big = 1;
    const int cols = epi == Epi::SWIGLU ? 128 : kBN;
    p.n_tiles = (N + cols - 1) / cols;
    const int64_t m_tiles = rows_upper / kBM + n_groups;
    p.grid = ((m_tiles * p.n_tiles + 7) / 8) * 8;
    return p;
}

// The router GEMM of a large batch (dense rows, fp32 out) on 256 x 256 tiles
// split along K, so that its few m-tiles make about 256 workgroups: a split of
// 2, 4 or 8 (at least 2, so that the partial-sum pass adds the bias), each
// slice at least 8 stages long. ksplit 0: the batch has too few rows (fewer
// than 32 tile rows of 256 rows) or K does not split; the caller takes
// another plan. The partial sums take ksplit x T rows, at most
// max(2 T, 131072) (with a split of 4 or 8, ksplit x m-tiles < 512).
GemmPlan plan_router_big(int64_t T, int N, int K) {
    GemmPlan p;
    p.bm = kBM;
    p.nw = 8;
    p.smajor = 0;
    p.big = 1;
    p.ksplit = 0;
    p.grid = 0;
    p.n_tiles = (N + kBN - 1) / kBN;
    const int64_t tiles = (T + kBM - 1) / kBM * p.n_tiles;
    if (tiles < 32) return p;
    int ks = 2;
    while (ks < 8 && tiles * ks < 256) ks *= 2;
    if (K % (ks * kKB) != 0 || K / ks < 8 * kKB) return p;
    p.ksplit = ks;
    p.grid = ((tiles * ks + 7) / 8) * 8;
    return p;
}

hipError_t launch_gemm_big(Epi epi, const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    if (p.grid == 0) return hipSuccess;
    if (a.K % kKB != 0 || a.N % 8 != 0 || a.ldc % 8 != 0) return hipErrorInvalidValue;
    GemmArgs b = a;
    b.ksplit = p.ksplit < 1 ? 1 : p.ksplit;
    // a K split: fp32 partial sums of dense rows (no groups, gather or shared
    // expert), every slice whole stages
    if (b.ksplit > 1 && (epi != Epi::PLAIN || !a.out_f32 || !a.partial || a.gather || a.sched || a.has_shared ||
                         a.K % (b.ksplit * kKB) != 0))
        return hipErrorInvalidValue;
    if (p.nw == 8)
        return epi == Epi::SWIGLU ? launch_big_epi<Epi::SWIGLU, 8>(b, p, s) : launch_big_epi<Epi::PLAIN, 8>(b, p, s);
    if (p.nw == 4)
        return epi == Epi::SWIGLU ? launch_big_epi<Epi::SWIGLU, 4>(b, p, s) : launch_big_epi<Epi::PLAIN, 4>(b, p, s);
    return hipErrorInvalidValue;
}

}  // namespace moe
