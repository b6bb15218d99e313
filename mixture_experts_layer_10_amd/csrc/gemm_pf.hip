// K5 / K6 at compute-bound shapes (bf16) on prepacked weights: the gate/up
// grouped GEMM with its fused SwiGLU and the routed down GEMM, 256 x 256
// tiles, the activation tile staged through a four-slot LDS ring and the
// weights streamed from HBM straight into registers.
//
// What it computes is that of gemm.hip (Perplexity "Lower latency and higher
// throughput with multi-node DeepSeek deployment", section "Roofline >
// GroupGEMM": per group, rows x weight^T; SWIGLU epilogue h = silu(gate) * up,
// infra guide "Data parallelism and expert parallelism", section 2.1). At
// prefill shapes (hundreds of rows per expert) the product is bound by the
// matrix cores, and what keeps them busy is hiding every load behind MFMAs:
//
//  * a workgroup of 4 wavefronts computes 256 rows x 4 weight panels of 64
//    rows (gate/up: 32 gate rows + the 32 up rows of the same h columns, 128
//    h columns per tile; down: 64 consecutive output columns, 256 per tile);
//    wavefront w owns panel w and all 256 rows,
//    as 8 x 2 fragments of v_mfma_f32_32x32x16_bf16 (256 accumulators, held
//    in the accumulation registers: one wavefront per SIMD);
//  * the weights come from the prepacked layout (moe_prepack_weights), in
//    which one wavefront's operand fragments of a 16-deep K step are 2 KB of
//    consecutive memory: two fully coalesced 16-byte loads per lane, issued
//    three K-stages (192 K) ahead into a four-stage register ring, never
//    through LDS;
//  * every load goes through a buffer descriptor: the base in scalar
//    registers, a 32-bit offset per lane, the stage offset in the scalar
//    offset (against 64-bit addresses per lane, a 64-bit add per load and
//    twice the address registers: gate/up 1-2% faster, 4 fewer spills);
//  * the activation rows (gathered through the dispatch permutation) go
//    HBM/L2 -> LDS by buffer_load_dwordx4 ... lds, K = 64 per stage (each row's
//    128 bytes one whole cache line), into a ring of four 32 KB slots, four
//    stages ahead (a slot is refilled as soon as the barrier after its last
//    read has passed);
//  * one barrier per stage, placed mid-stage, that waits only for the loads
//    the next stage needs (vmcnt counts outstanding loads in issue order), so
//    loads issued later stay in flight across it; the MFMAs of the stage's
//    last two K steps run while the next stage's first fragments are read;
//  * 16-byte granule q of LDS row r sits at q ^ ((r >> 1) & 7): the fragment
//    reads (32 rows x one granule per lane half) are free of bank conflicts;
//  * a group's rows are split evenly over its m-tiles; the K loop is
//    instantiated for each count of 32-row blocks with data (1..8), so a
//    tile reads and multiplies only its own blocks with no branch in the
//    loop, and scheduling groups fix the order of each K step's MFMAs,
//    fragment reads and loads;
//  * the MFMAs take the weights as their first operand, so the accumulators
//    hold the transposed tile: a lane holds one row and runs of four
//    consecutive columns, and the epilogue (h = silu(gate) * up, or the down
//    GEMM's outputs as they are) stages the tile in the idle LDS ring with
//    one 8-byte write per four outputs (four times fewer LDS writes than a
//    column per lane: the layer 0.4% faster, mostly in the down GEMM) and
//    writes whole 16-byte pieces of rows.
#include <utility>

#include "gemm_tile.h"

namespace moe {
namespace {

constexpr int kBM = 256;                 // rows per tile
constexpr int kNW = 4;                   // wavefronts (one weight panel each)
constexpr int kNT = kNW * 64;            // threads
constexpr int kKB = 64;                  // K per stage
constexpr int kRowB = kKB * 2;           // LDS bytes per row per stage
constexpr int kGran = kRowB / 16;        // 16-byte granules per row
constexpr int kSlots = 4;                // LDS ring
constexpr int kSlotB = kBM * kRowB;      // 32 KB
constexpr int kALoads = kBM * kGran / kNT;       // direct loads per thread per stage (8)
constexpr int kRowsPerLoad = 64 / kGran;         // rows one direct load instruction fills (8)
constexpr int kKSteps = kKB / 16;                // MFMA K steps per stage (4)
constexpr int kFragB = 1024;                     // bytes of one 32 x 16 operand fragment
constexpr int kStepB = 2 * kFragB;               // packed bytes of a panel per K step

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 frag(const vec16& v) { return __builtin_bit_cast(bf16x8, v); }



// s_waitcnt immediate (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]).
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

template <Epi EPI>
__global__ __launch_bounds__(kNT, 1) void gemm_pf_kernel(GemmArgs a, int n_tiles) {
    // The LDS ring as four separate arrays, each indexed only by a constant
    // slot number: the compiler then knows that a fragment read of one slot
    // cannot alias a direct load into another, and does not make the read
    // wait for every direct load in flight.
    __shared__ __attribute__((aligned(16))) unsigned char s_a0[kSlotB], s_a1[kSlotB], s_a2[kSlotB], s_a3[kSlotB];
    auto slot = [&](auto u_c) __attribute__((always_inline)) -> unsigned char* {
        constexpr int U = decltype(u_c)::value % kSlots;
        return U == 0 ? s_a0 : U == 1 ? s_a1 : U == 2 ? s_a2 : s_a3;
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    Tile tl;
    if (!find_tile(a, n_tiles, kBM, tl, /*balanced=*/true)) return;
    const int g = tl.g, nt = tl.nt;
    const bool shared = tl.shared;
    const int row0 = tl.row0, m0 = tl.m0, rows = tl.rows;
    const int K = a.K;
    const int nkb = K / kKB;
    const int last = nkb - 1;
    const int nrb = (rows + 31) >> 5;                 // 32-row blocks with data (uniform)

    // ---- activation rows: load j of wavefront w fills rows (4 j + w) * 8 +
    // lane / 8 of the slot, granule position lane % 8, with the granule the
    // swizzle puts there. The gathered source rows are looked up with all
    // eight permutation loads in flight together. ------------------------------
    const int lrow = lane / kGran;
    const unsigned char* Ag = static_cast<const unsigned char*>(shared ? a.A_shared : a.A);
    int rsl[kALoads];
    uint32_t src[kALoads];
#pragma unroll
    for (int j = 0; j < kALoads; ++j) {
        const int rs = (kNW * j + wave) * kRowsPerLoad + lrow;
        rsl[j] = rs;
        src[j] = static_cast<uint32_t>(rs < rows ? rs : rows - 1);   // rows past the end: a valid row, unused
    }
    if (shared) {
#pragma unroll
        for (int j = 0; j < kALoads; ++j) src[j] += m0;
    } else if (a.gather) {
        int pv[kALoads];
#pragma unroll
        for (int j = 0; j < kALoads; ++j) pv[j] = a.perm[row0 + m0 + static_cast<int>(src[j])];
#pragma unroll
        for (int j = 0; j < kALoads; ++j) src[j] = static_cast<uint32_t>(pv[j] / a.topk);
    } else {
#pragma unroll
        for (int j = 0; j < kALoads; ++j) src[j] += row0 + m0;
    }
    uint32_t aoff[kALoads];
#pragma unroll
    for (int j = 0; j < kALoads; ++j)
        aoff[j] = src[j] * static_cast<uint32_t>(K * 2) + (((lane % kGran) ^ swz(rsl[j])) * 16);

    // ---- weights: this wavefront's panel of the packed layout ----------------
    // A panel past the last one (N not a multiple of the tile) reads the last
    // panel; its results are dropped.
    const int n_panels = EPI == Epi::SWIGLU ? a.inter / 32 : a.N / 64;
    int panel = nt * kNW + wave;
    panel = panel < n_panels ? panel : n_panels - 1;
    const unsigned char* Bw = static_cast<const unsigned char*>(shared ? a.B_shared : a.B) +
                              (shared ? int64_t{0} : static_cast<int64_t>(g) * a.b_stride * 2) +
                              static_cast<int64_t>(panel) * (K / 16) * kStepB;
    const uint32_t boff = static_cast<uint32_t>(lane) * 16;
    // The panel through a buffer descriptor (K / 16 steps of 2 KB): a load
    // then sends 32-bit lane offsets, and the stage offset rides in a scalar.
    const __amdgpu_buffer_rsrc_t bres = byte_buffer(Bw, static_cast<uint32_t>(K / 16) * kStepB);

    // The activation rows through a buffer descriptor too (offsets below
    // 4 GiB: the operand size limit): 32-bit row offsets, the stage offset
    // in a scalar.
    const __amdgpu_buffer_rsrc_t ares = byte_buffer(Ag, 0xFFFFFFFFu);
    // A(kb) -> slot kb % 4 (kb past the end: the last stage again, into a
    // slot nobody reads any more)
    auto issue_a = [&](auto u_c, int kb) __attribute__((always_inline)) {
        const int kc = kb < last ? kb : last;
        unsigned char* sa = slot(u_c);
#pragma unroll
        for (int j = 0; j < kALoads; ++j)
            buf_load_lds16(ares, aoff[j], kc * kRowB, sa + (kNW * j + wave) * kRowsPerLoad * kRowB);
    };
    // B register ring: four stages x 4 K steps x (gate/low, up/high) halves;
    // B(kb) -> ring slot kb % 4.
    vec16 br[4][kKSteps][2];
    auto issue_b = [&](auto u_c, int kb) __attribute__((always_inline)) {
        constexpr int S = decltype(u_c)::value % 4;
        const int kc = kb < last ? kb : last;
        const int so = kc * kKSteps * kStepB;
#pragma unroll
        for (int t = 0; t < kKSteps; ++t) {
            // load 2 t + h at byte 1024 (2 t + h) of the stage: below 4096 in
            // the instruction's offset field, the rest in the scalar offset
            br[S][t][0] = buf_ld16(bres, boff + (t % 2) * kStepB, so + (t / 2) * 2 * kStepB);
            br[S][t][1] = buf_ld16(bres, boff + (t % 2) * kStepB + kFragB, so + (t / 2) * 2 * kStepB);
        }
    };
    // One load of A(kb) or B(kb) (load j of the stage's eight), for issuing
    // the loads one at a time between MFMAs.
    auto issue_a_one = [&](auto u_c, auto j_c, int kb) __attribute__((always_inline)) {
        constexpr int J = decltype(j_c)::value;
        const int kc = kb < last ? kb : last;
        buf_load_lds16(ares, aoff[J], kc * kRowB, slot(u_c) + (kNW * J + wave) * kRowsPerLoad * kRowB);
    };
    auto issue_b_one = [&](auto u_c, auto j_c, int kb) __attribute__((always_inline)) {
        constexpr int S = decltype(u_c)::value % 4;
        constexpr int J = decltype(j_c)::value;
        const int kc = kb < last ? kb : last;
        br[S][J / 2][J % 2] = buf_ld16(bres, boff + (J % 4) * kFragB, kc * kKSteps * kStepB + (J / 4) * 4 * kFragB);
    };

    // ---- fragment reads: lane l reads row l % 32 of a 32-row block, granule
    // 2 t + l / 32 of K step t ------------------------------------------------
    const int fr = lane & 31;
    int f_off[kKSteps];
#pragma unroll
    for (int t = 0; t < kKSteps; ++t) f_off[t] = fr * kRowB + (((2 * t + (lane >> 5)) ^ swz(fr)) * 16);

    f32x16 acc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i][0] = acc[i][1] = f32x16{};

    // Wait until at most VM loads of this thread are outstanding (and, with
    // LGKM, its LDS reads are done), then, with BAR, a bare barrier (no
    // fence: the fills are waited for explicitly). The empty asm statements
    // keep the compiler from moving memory accesses across it, the scheduling
    // barriers keep MFMAs on their side of it.
    auto wait = [&](auto vm_c, auto bar_c) __attribute__((always_inline)) {
        constexpr bool BAR = decltype(bar_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(decltype(vm_c)::value, BAR ? 0 : 15));
        asm volatile("" ::: "memory");
        if constexpr (BAR) {
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
    using Yes = std::true_type;
    using No = std::false_type;
    constexpr int kGroup = 2 * kALoads;                             // loads of one stage (A and B: 8 each)

    // ---- pipeline -----------------------------------------------------------
    // Iteration j issues B(j + 3), then, after its mid-stage barrier, A(j + 4);
    // the prologue stands in for iterations -4..-1. Iteration j (stage j in
    // LDS slot j % 4 and ring slot j % 4; K step 0's fragments already read):
    //   wait for B(j)  [after it: A(j+1), B(j+1), A(j+2), B(j+2), A(j+3)]  vmcnt(40)
    //   K steps 0, 1 and 2, each with the fragment reads of the next step;
    //   B(j+3) (ring slot (j-1) % 4, last read by stage j-1) is issued
    //   three loads in step 0, three in step 1 and two in step 2 (all eight
    //   in step 0: gate/up 6.3% slower; two per step with the last two after
    //   the barrier, four per step with A(j+4) split over step 3 and the next
    //   step 0, or 4-4-0 or 2-3-3 over steps 0-2: no better);
    //   wait for A(j+1) [after it: B(j+1), A(j+2), B(j+2), A(j+3), B(j+3)] vmcnt(40)
    //   and this thread's LDS reads, then barrier: A(j+1) has landed for
    //   every wavefront and nobody reads slot j % 4 any more;
    //   K step 3 with A(j+4) (into slot j % 4) issued during it, and the reads
    //   of step 0 of stage j+1.
    // Loads past the last stage re-read it into free slots, so the wait
    // counts hold to the end.
    issue_a(C0{}, 0);
    issue_b(C0{}, 0);
    issue_a(C1{}, 1);
    issue_b(C1{}, 1);
    issue_a(C2{}, 2);
    issue_b(C2{}, 2);
    issue_a(C3{}, 3);
    wait(std::integral_constant<int, 3 * kGroup>{}, Yes{});         // A(0) for every wavefront

    // The K loop for a tile of NRB 32-row blocks with data (1..8): only those
    // blocks are read and multiplied, so the loop is branch-free, and
    // scheduling groups lay out each K step explicitly. In a step the NRB
    // fragment reads of the next step follow every second of the step's 2 NRB
    // MFMAs (the compiler then waits for each only at the next step), and the
    // stage's loads, where the step issues any, follow every second MFMA of
    // the second half (step 3's over the whole step). With one wavefront per
    // SIMD a load or read holds up the wavefront's issue while its addresses
    // are taken in, which an MFMA in flight hides; and the barrier keeps the
    // four wavefronts in step, so what a step issues reaches the CU's address
    // unit and LDS together: few per step, spread out. (Measured, prefill
    // layer: the weight loads all in step 0 against 3-3-2 over steps 0-2
    // 4.3% slower; the reads one per MFMA in the first half against one per
    // two MFMAs over the step about 1%; with the reads so spread the kernel
    // spills 12 registers instead of 36.)
    // Left to itself, the compiler bunched the loads and read each fragment
    // just before its MFMA, waiting on every read.
    using L4 = std::integral_constant<int, 0>;
    using H4 = std::integral_constant<int, 4>;
    auto kloop = [&](auto nrb_c) __attribute__((always_inline)) {
        constexpr int NRB = decltype(nrb_c)::value;
        bf16x8 af[2][NRB];
        auto read = [&](auto u_c, auto t_c) __attribute__((always_inline)) {
            constexpr int T = decltype(t_c)::value;
            const unsigned char* st = slot(u_c) + f_off[T];
#pragma unroll
            for (int i = 0; i < NRB; ++i) af[T % 2][i] = frag(ld16(st + i * 32 * kRowB));
        };
        // the MFMAs of K step t for row blocks [I0, I0 + 4) (those below
        // NRB); after each block, ld(i) issues load i of the stage
        auto mfma = [&](auto u_c, auto t_c, auto i0_c, auto ld) __attribute__((always_inline)) {
            constexpr int S = decltype(u_c)::value % 4;
            constexpr int T = decltype(t_c)::value;
            constexpr int I0 = decltype(i0_c)::value;
            auto block = [&](auto i_c) __attribute__((always_inline)) {
                constexpr int i = decltype(i_c)::value;
                if constexpr (i < NRB) {
                    // weights as the first operand: the accumulators hold the
                    // transposed tile (see the epilogue)
                    acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(br[S][T][0]), af[T % 2][i], acc[i][0], 0, 0, 0);
                    acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(br[S][T][1]), af[T % 2][i], acc[i][1], 0, 0, 0);
                }
                ld(i_c);
            };
            block(std::integral_constant<int, I0>{});
            block(std::integral_constant<int, I0 + 1>{});
            block(std::integral_constant<int, I0 + 2>{});
            block(std::integral_constant<int, I0 + 3>{});
        };
        auto none = [](auto) __attribute__((always_inline)) {};
        // scheduling groups of one K step (mask 0x008 MFMA, 0x100 LDS read,
        // 0x010 VMEM): the step's NRB fragment reads after every second of its
        // 2 NRB MFMAs, and its LD loads (0: none) after every second MFMA of
        // the second half
        auto groups = [&](auto loads_c) __attribute__((always_inline)) {
            constexpr int LD = decltype(loads_c)::value;
            constexpr int ST = (2 * LD <= NRB) ? 2 : 1;
#pragma unroll
            for (int m = 0; m < 2 * NRB; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (m % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                const int q = m - NRB;
                if (LD > 0 && q >= 0 && (q + 1) % ST == 0 && (q + 1) / ST <= LD)
                    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
            }
            constexpr int DONE = LD > 0 ? (NRB / ST < LD ? NRB / ST : LD) : 0;
            if constexpr (LD > DONE) __builtin_amdgcn_sched_group_barrier(0x010, LD - DONE, 0);
        };
        // a step's 2 NRB MFMAs, the first NRB each followed by a fragment
        // read, and its LD loads spread evenly over all of them
        auto groups_full = [&](auto loads_c) __attribute__((always_inline)) {
            constexpr int LD = decltype(loads_c)::value;
#pragma unroll
            for (int q = 0; q < 2 * NRB; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (q % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                // load k after MFMA (k + 1) * 2 NRB / LD - 1
                if (LD > 0 && ((q + 1) * LD) / (2 * NRB) > (q * LD) / (2 * NRB))
                    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
            }
        };
        auto iteration = [&](auto u_c, int kb) __attribute__((always_inline)) {
            constexpr int U = decltype(u_c)::value;
            using N = std::integral_constant<int, (U + 1) % 4>;
            using P = std::integral_constant<int, (U + 3) % 4>;
            // B(j+3)'s eight loads spread over K steps 0, 1 and 2 (3, 3, 2),
            // each after a block of the step's second half (all of them were
            // issued by the wait for A(j+1), so its count holds)
            auto ldb_at = [&](auto base_c, auto cnt_c) __attribute__((always_inline)) {
                return [&, base_c, cnt_c](auto i_c) __attribute__((always_inline)) {
                    constexpr int Q = decltype(i_c)::value - 4;
                    if constexpr (Q >= 0 && Q < decltype(cnt_c)::value)
                        issue_b_one(P{}, std::integral_constant<int, decltype(base_c)::value + Q>{}, kb + 3);
                };
            };
            // only the loads of the tile's NRB blocks: load J of every
            // wavefront fills rows 32 J .. 32 J + 31 of the slot
            auto lda = [&](auto j_c) __attribute__((always_inline)) {
                if constexpr (decltype(j_c)::value < NRB) issue_a_one(u_c, j_c, kb + 4);
            };
            // B(j): after it A(j+1), B(j+1), A(j+2), B(j+2), A(j+3). In the
            // first iterations the prologue's A stages hold all eight loads,
            // so these counts then wait for more than B(j): never less.
            wait(std::integral_constant<int, 3 * NRB + 2 * kALoads>{}, No{});
            mfma(u_c, C0{}, L4{}, none);
            read(u_c, C1{});
            mfma(u_c, C0{}, H4{}, ldb_at(std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{}));
            mfma(u_c, C1{}, L4{}, none);
            read(u_c, C2{});
            mfma(u_c, C1{}, H4{}, ldb_at(std::integral_constant<int, 3>{}, std::integral_constant<int, 3>{}));
            mfma(u_c, C2{}, L4{}, none);
            read(u_c, C3{});
            mfma(u_c, C2{}, H4{}, ldb_at(std::integral_constant<int, 6>{}, std::integral_constant<int, 2>{}));
            groups(std::integral_constant<int, 3>{});
            groups(std::integral_constant<int, 3>{});
            groups(std::integral_constant<int, 2>{});
            // A(j+1) for every wavefront: after it B(j+1), A(j+2), B(j+2), A(j+3), B(j+3)
            wait(std::integral_constant<int, 3 * kALoads + 2 * NRB>{}, Yes{});
            mfma(u_c, C3{}, L4{}, lda);
            read(N{}, C0{});
            mfma(u_c, C3{}, H4{}, lda);
            groups_full(std::integral_constant<int, NRB>{});
            __builtin_amdgcn_sched_barrier(0);
        };
        read(C0{}, C0{});
        // Whole groups of four stages with no conditional code; then the
        // last zero to three stages.
        int kb = 0;
        for (; kb + 4 <= nkb; kb += 4) {
            iteration(C0{}, kb);
            iteration(C1{}, kb + 1);
            iteration(C2{}, kb + 2);
            iteration(C3{}, kb + 3);
        }
        if (kb < nkb) iteration(C0{}, kb);
        if (kb + 1 < nkb) iteration(C1{}, kb + 1);
        if (kb + 2 < nkb) iteration(C2{}, kb + 2);
    };
    switch (nrb) {
        case 1: kloop(std::integral_constant<int, 1>{}); break;
        case 2: kloop(std::integral_constant<int, 2>{}); break;
        case 3: kloop(std::integral_constant<int, 3>{}); break;
        case 4: kloop(std::integral_constant<int, 4>{}); break;
        case 5: kloop(std::integral_constant<int, 5>{}); break;
        case 6: kloop(std::integral_constant<int, 6>{}); break;
        case 7: kloop(std::integral_constant<int, 7>{}); break;
        default: kloop(std::integral_constant<int, 8>{}); break;
    }
    // no direct-load write may outlive the loop: the epilogue reuses the ring
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __syncthreads();

    // ---- epilogue: the MFMAs took the weights as their first operand, so
    // each 32 x 32 accumulator fragment is the transposed output block: lane
    // l holds tile row l % 32 and, for q = 0..3, the four consecutive output
    // columns 8 q + 4 (l / 32) + (0..3). Those four are rounded to bf16 (h =
    // silu(gate) * up formed first) and staged with one 8-byte LDS write,
    // 64 rows per LDS slot, as a row-major tile whose 16-byte granules are
    // XOR-swizzled by the row (so the 32 rows a write covers fall on all
    // banks); the workgroup then writes whole 16-byte pieces of rows. ----
    const int64_t crow0 = shared ? m0 : static_cast<int64_t>(row0) + m0;
    unsigned char* Cb = static_cast<unsigned char*>(shared ? a.C_shared : a.C);
    const int lc = lane & 31, lh = lane >> 5;
    constexpr int TC = (EPI == Epi::SWIGLU ? 32 : 64) * kNW;          // output columns of the tile
    constexpr int PRB = TC * 2;                                       // staged bytes per row
    constexpr int GPR = PRB / 16;                                     // 16-byte granules per row
    static_assert(64 * PRB <= kSlotB, "64 staged rows per slot");
    static_assert(64 % GPR == 0, "the swizzle of a row is that of its row in the slot");
    auto put = [&](auto i_c) __attribute__((always_inline)) {
        constexpr int I = decltype(i_c)::value;
        if (I < nrb) {
            unsigned char* sl = slot(std::integral_constant<int, I / 2>{});
            const int r = (I % 2) * 32 + lc;                          // row within the slot
            unsigned char* row = sl + r * PRB + lh * 8;
            const int sw = r % GPR;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (EPI == Epi::SWIGLU) {
                    const int g = wave * 4 + q;                       // granule of columns 32 w + 8 q ..
                    const float h0 = silu_mul(acc[I][0][4 * q + 0], acc[I][1][4 * q + 0]);
                    const float h1 = silu_mul(acc[I][0][4 * q + 1], acc[I][1][4 * q + 1]);
                    const float h2 = silu_mul(acc[I][0][4 * q + 2], acc[I][1][4 * q + 2]);
                    const float h3 = silu_mul(acc[I][0][4 * q + 3], acc[I][1][4 * q + 3]);
                    *reinterpret_cast<uint2*>(row + ((g ^ sw) * 16)) = uint2{pack_bf16x2(h0, h1), pack_bf16x2(h2, h3)};
                } else {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int g = wave * 8 + hh * 4 + q;          // granule of columns 64 w + 32 hh + 8 q ..
                        *reinterpret_cast<uint2*>(row + ((g ^ sw) * 16)) =
                            uint2{pack_bf16x2(acc[I][hh][4 * q + 0], acc[I][hh][4 * q + 1]),
                                  pack_bf16x2(acc[I][hh][4 * q + 2], acc[I][hh][4 * q + 3])};
                    }
                }
            }
        }
    };
    put(std::integral_constant<int, 0>{});
    put(std::integral_constant<int, 1>{});
    put(std::integral_constant<int, 2>{});
    put(std::integral_constant<int, 3>{});
    put(std::integral_constant<int, 4>{});
    put(std::integral_constant<int, 5>{});
    put(std::integral_constant<int, 6>{});
    put(std::integral_constant<int, 7>{});
    __syncthreads();
    // N and ldc are multiples of 8 (checked at launch), so a 16-byte piece
    // lies wholly inside or wholly past the output's columns.
    const int c0 = nt * TC;
    for (int q = tid; q < rows * GPR; q += kNT) {
        const int r = q / GPR, gq = q % GPR;
        const int col = c0 + gq * 8;
        const unsigned char* sl = r < 64 ? s_a0 : r < 128 ? s_a1 : r < 192 ? s_a2 : s_a3;
        if (col < a.N)
            st16(Cb + ((crow0 + r) * a.ldc + col) * 2,
                 *reinterpret_cast<const vec16*>(sl + (r & 63) * PRB + ((gq ^ (r % GPR)) * 16)));
    }
}

// Packed layout of a gate/up weight [2I, K] (moe_prepack_weights): element
// (row n, column k) of panel p, half h (gate rows 32p.., up rows I + 32p..)
// sits at byte ((p * K/16 + k/16) * 2 + h) * 1024 + l * 16 + (k % 8) * 2 with
// lane l = (n - first row of the half) + 32 * ((k / 8) % 2).
__global__ __launch_bounds__(256) void prepack_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                      int64_t n_chunks, int K, int half_off, int pstride) {
    // one thread per 16-byte packed chunk: (panel, k step, half, lane)
    for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < n_chunks;
         c += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int l = static_cast<int>(c & 63);
        const int h = static_cast<int>((c >> 6) & 1);
        const int64_t ps = c >> 7;                   // panel * K/16 + k step
        const int ksteps = K / 16;
        const int64_t p = ps / ksteps;
        const int s = static_cast<int>(ps - p * ksteps);
        const int64_t n = h * half_off + p * pstride + (l & 31);
        const int k = s * 16 + (l >> 5) * 8;
        st16(dst + c * 8, ld16(src + n * K + k));
    }
}

}  // namespace

GemmPlan plan_gemm_pf(int64_t rows_upper, int n_groups, int inter) {
    GemmPlan p = plan_gemm_big(Epi::SWIGLU, rows_upper, n_groups, inter);
    p.nw = kNW;
    p.big = 2;
    return p;
}

hipError_t launch_gemm_pf(Epi epi, const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    if (p.grid == 0) return hipSuccess;
    if (a.K % kKB != 0 || a.N % 8 != 0 || a.ldc % 8 != 0) return hipErrorInvalidValue;
    if (epi == Epi::SWIGLU ? a.inter % 32 != 0 : (a.N % 64 != 0 || a.out_f32 || a.gather)) return hipErrorInvalidValue;
    GemmArgs b = a;
    b.ksplit = 1;
    if (epi == Epi::SWIGLU)
        hipLaunchKernelGGL(gemm_pf_kernel<Epi::SWIGLU>, dim3(static_cast<unsigned>(p.grid)), dim3(kNT), 0, s, b, p.n_tiles);
    else
        hipLaunchKernelGGL(gemm_pf_kernel<Epi::PLAIN>, dim3(static_cast<unsigned>(p.grid)), dim3(kNT), 0, s, b, p.n_tiles);
    return hipGetLastError();
}

hipError_t launch_prepack(const void* src, void* dst, int64_t n_experts, int inter, int K, hipStream_t s) {
    const int64_t per = static_cast<int64_t>(2 * inter) * K / 8;      // 16-byte chunks per expert
    for (int64_t e = 0; e < n_experts; ++e) {
        const int64_t blocks = std::min<int64_t>((per + 255) / 256, 8192);
        hipLaunchKernelGGL(prepack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                           static_cast<const uint16_t*>(src) + e * 2 * inter * K,
                           static_cast<uint16_t*>(dst) + e * 2 * inter * K, per, K, inter, 32);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t launch_prepack_down(const void* src, void* dst, int64_t n_experts, int N, int K, hipStream_t s) {
    const int64_t per = static_cast<int64_t>(N) * K / 8;              // 16-byte chunks per expert
    for (int64_t e = 0; e < n_experts; ++e) {
        const int64_t blocks = std::min<int64_t>((per + 255) / 256, 8192);
        hipLaunchKernelGGL(prepack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                           static_cast<const uint16_t*>(src) + e * static_cast<int64_t>(N) * K,
                           static_cast<uint16_t*>(dst) + e * static_cast<int64_t>(N) * K, per, K, 32, 64);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace moe
