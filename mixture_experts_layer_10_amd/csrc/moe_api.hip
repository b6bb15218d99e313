// The C ABI of libmoe.so: argument validation, workspace layout, and the
// launch sequence of each stage. Host code only; kernels live in route.hip,
// dispatch.hip, gemm.hip, quant.hip and combine.hip.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <unordered_map>
#include <vector>

#include <hip/hip_runtime.h>

#include "moe_internal.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int validate(const moe_config* c) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (c->abi_version != MOE_ABI_VERSION) return MOE_ERR_ABI_MISMATCH;
    if (c->hidden <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->inter <= 0 || c->shared_inter < 0)
        return MOE_ERR_INVALID_ARG;
    if (c->n_group <= 0 || c->n_experts % c->n_group != 0) return MOE_ERR_INVALID_ARG;
    if (c->topk_group <= 0 || c->topk_group > c->n_group) return MOE_ERR_INVALID_ARG;
    if (c->top_k > c->topk_group * (c->n_experts / c->n_group)) return MOE_ERR_INVALID_ARG;
    // a group is scored by the sum of its two best experts: it needs two
    if (c->n_group > 1 && c->n_experts / c->n_group < 2) return MOE_ERR_INVALID_ARG;
    if (c->expert_begin < 0 || c->expert_end <= c->expert_begin || c->expert_end > c->n_experts)
        return MOE_ERR_INVALID_ARG;
    if (c->score_fn != MOE_SCORE_SOFTMAX && c->score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
    if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_INVALID_ARG;
    if (!isfinite(c->routed_scale) || !isfinite(c->capacity_factor)) return MOE_ERR_INVALID_ARG;
    if (c->dtype != MOE_DTYPE_F32 && c->dtype != MOE_DTYPE_BF16 && c->dtype != MOE_DTYPE_FP8 &&
        c->dtype != MOE_DTYPE_MXFP4)
        return MOE_ERR_INVALID_ARG;
    if (c->out_dtype != MOE_DTYPE_F32 && c->out_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
    // Valid, but outside what the kernels are built for.
    if (c->top_k > 16 || c->n_experts > 512 || c->n_group > 64) return MOE_ERR_UNSUPPORTED;
    if (c->expert_end - c->expert_begin > 1024) return MOE_ERR_UNSUPPORTED;
    if (c->hidden % 128 != 0 || c->inter % 128 != 0 || c->shared_inter % 128 != 0) return MOE_ERR_UNSUPPORTED;
    // The FP4 GEMM reduces K in chunks of 256 (one 128-byte line per weight row).
    if (c->dtype == MOE_DTYPE_MXFP4 && (c->hidden % 256 != 0 || c->inter % 256 != 0 || c->shared_inter % 256 != 0))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int act_bytes(const moe_config* c) { return c->dtype == MOE_DTYPE_F32 ? 4 : c->dtype == MOE_DTYPE_BF16 ? 2 : 1; }
int row_bytes(const moe_config* c) { return c->dtype == MOE_DTYPE_F32 ? 4 : 2; }

// The GEMM kernels address a row of an operand as row * K * element bytes in
// 32 bits (the base pointer carries the rest), so no operand they read may
// span more than 4 GiB: the gathered hidden states x [T, H], the intermediate rows
// h [T k, I] and h_shared [T, I_s], the router weight [E, H] and one
// expert's stacked weights [2 I, H] (bf16 bytes for the e4m3 and FP4 paths,
// which is an upper bound of their own). `router_only`: the router GEMM's
// operands alone.
bool offsets_fit(const moe_config* c, int64_t T, bool router_only) {
    const int64_t eb = c->dtype == MOE_DTYPE_F32 ? 4 : 2;
    const int64_t lim = int64_t{1} << 32;
    const int64_t H = c->hidden;
    int64_t need = std::max(T * H, static_cast<int64_t>(c->n_experts) * H);
    if (!router_only) {
        need = std::max(need, T * c->top_k * static_cast<int64_t>(c->inter));
        need = std::max(need, T * static_cast<int64_t>(c->shared_inter));
        need = std::max(need, 2 * static_cast<int64_t>(std::max(c->inter, c->shared_inter)) * H);
    }
    return need * eb <= lim;     // the last row starts below 4 GiB and ends at most there
}
Elem gemm_elem(const moe_config* c) { return c->dtype == MOE_DTYPE_F32 ? Elem::F32 : Elem::BF16; }

// Expert GEMMs on e4m3 activations: FP8 block-scaled or MX (FP4 weights).
bool quantised(const moe_config* c) { return c->dtype == MOE_DTYPE_FP8 || c->dtype == MOE_DTYPE_MXFP4; }
GemmPlan plan_quantised(const moe_config* c, Epi epi, int64_t rows_upper, int n_groups, int64_t per_group, int N) {
    return c->dtype == MOE_DTYPE_MXFP4 ? plan_gemm_mx(epi, rows_upper, n_groups, per_group, N)
                                      : plan_gemm_fp8(epi, rows_upper, n_groups, per_group, N);
}
hipError_t launch_quantised(const moe_config* c, Epi epi, const GemmArgs& a, const GemmPlan& p, hipStream_t s) {
    return c->dtype == MOE_DTYPE_MXFP4 ? launch_gemm_mx(epi, a, p, s) : launch_gemm_fp8(epi, a, p, s);
}

// Workspace layout for up to T tokens; every region 256-byte aligned.
struct Layout {
    size_t status;                      // the error word of moe_dispatch_errors (offset 0)
    size_t logits, ids, w, raw, counts, offsets, perm, inv, chunk_hist, chunk_base, chunk_bad, sched, tiles, partial;
    size_t h, h_shared, rows, shared_out;
    size_t xq, xs, hs, hs_shared;       // FP8, MXFP4: quantised x and the scales of x and h
    size_t total;
};

// The workspace opens with a status region; its first int32 is the error
// word: expert ids outside [0, E) met by the last dispatch on the workspace.
constexpr size_t kStatusBytes = 256;

int router_chunk(const moe_config* c) { return c->dtype == MOE_DTYPE_F32 ? 64 : 128; }

// The routed GEMMs' plan (bf16 and fp32 layers). With prepacked bf16 weights
// the 256 x 256 packed tiles pay from about 32 rows per expert, where the
// LDS-staged canonical tiles need about 256 (plan_gemm): measured on the EP8
// decode share (32 of 256 experts), per layer, 1024 tokens (32 rows per
// expert) 0.684 against 0.734 ms, 2048 tokens 0.770 against 0.820 ms, 4096
// tokens 1.085 against 1.409 ms. The packed down GEMM gains most (2048
// tokens: 0.245 against 0.284 ms, the shared expert's down beside it 0.197
// against 0.270).
GemmPlan routed_plan(const moe_config* c, Epi epi, int64_t P, int El, int64_t per_expert, int N, bool packed) {
    GemmPlan p = plan_gemm(gemm_elem(c), epi, P, El, per_expert, N);
    if (!p.big && packed && c->dtype == MOE_DTYPE_BF16 && per_expert >= 32) {
        const GemmPlan b = plan_gemm_big(epi, P, El, N);
        if ((P / 256) * b.n_tiles >= 512) p = b;
    }
    return p;
}

// Entries of the tile tables of the routed 256 x 256 launches for a batch of
// T tokens: the gate/up launch's upper-bound grid, then the down launch's,
// and 0 when the routed GEMMs do not take 256 x 256 tiles. Non-decreasing in
// T (a workspace sized for T serves every smaller batch).
int64_t big_tile_entries(const moe_config* c, int64_t T) {
    if (c->dtype != MOE_DTYPE_BF16) return 0;
    const int64_t El = c->expert_end - c->expert_begin, P = T * c->top_k;
    const int64_t per_expert = (P + c->n_experts - 1) / c->n_experts;
    // sized for a caller with packed weights (the larger of the two plans)
    const GemmPlan p1 = routed_plan(c, Epi::SWIGLU, P, static_cast<int>(El), per_expert, static_cast<int>(c->inter), true);
    if (!p1.big) return 0;
    return p1.grid + plan_gemm_big(Epi::PLAIN, P, static_cast<int>(El), static_cast<int>(c->hidden)).grid;
}

// Rows of router partial sums for any batch up to T: the split-K plan of the
// decode tiles, or, for a bf16 batch of 32 or more 256-row tiles, that of
// the 256 x 256 tiles (at most max(2 T, 131072) rows).
int64_t router_partial_rows_upto(const moe_config* c, int64_t T) {
    int64_t rows = splitk_partial_rows_upto(T, c->n_experts, c->hidden, router_chunk(c));
    if (gemm_elem(c) == Elem::BF16 && (T + 255) / 256 * ((c->n_experts + 255) / 256) >= 32)
        rows = std::max(rows, std::max<int64_t>(2 * T, 131072));
    return rows;
}

Layout layout(const moe_config* c, int64_t T) {
    const int64_t E = c->n_experts, El = c->expert_end - c->expert_begin, k = c->top_k;
    const int64_t P = T * k;
    // scratch whose need can fall as T grows is sized for the largest need
    // of any batch up to T, so a workspace sized for T serves them all
    const int64_t nchunk = dispatch_chunks_upto(P);
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align_up(bytes);
        return at;
    };
    L.status = take(kStatusBytes);
    L.logits = take(sizeof(float) * T * E);
    L.ids = take(sizeof(int32_t) * P);
    L.w = take(sizeof(float) * P);
    L.raw = take(sizeof(int32_t) * El);
    L.counts = take(sizeof(int32_t) * El);
    L.offsets = take(sizeof(int32_t) * (El + 1));
    L.perm = take(sizeof(int32_t) * P);
    L.inv = take(sizeof(int32_t) * P);
    L.chunk_hist = take(sizeof(int32_t) * nchunk * El);
    L.chunk_base = take(sizeof(int32_t) * nchunk * El);
    L.chunk_bad = take(sizeof(int32_t) * nchunk);
    L.sched = take(sizeof(int32_t) * (El + 2 + 2 * 9));    // m-tile prefix, then two sets of XCD ranges
    L.tiles = take(sizeof(int32_t) * 4 * big_tile_entries(c, T));
    L.partial = take(sizeof(float) * router_partial_rows_upto(c, T) * E);
    L.h = take(static_cast<size_t>(act_bytes(c)) * P * c->inter);
    L.h_shared = take(static_cast<size_t>(act_bytes(c)) * T * c->shared_inter);
    L.rows = take(static_cast<size_t>(row_bytes(c)) * P * c->hidden);
    L.shared_out = take(sizeof(float) * T * c->hidden);
    // scale bytes per activation element: FP8 one float per 128, MXFP4 one byte per 32
    const bool fp8 = c->dtype == MOE_DTYPE_FP8, mx = c->dtype == MOE_DTYPE_MXFP4;
    auto sbytes = [&](int64_t rows, int64_t cols) -> size_t {
        return fp8 ? sizeof(float) * rows * (cols / 128) : mx ? static_cast<size_t>(rows) * (cols / 32) : 0;
    };
    L.xq = take(fp8 || mx ? static_cast<size_t>(T) * c->hidden : 0);
    L.xs = take(sbytes(T, c->hidden));
    L.hs = take(sbytes(P, c->inter));
    L.hs_shared = take(sbytes(T, c->shared_inter));
    L.total = off;
    return L;
}

// The packed weight buffer of moe_prepack_weights (bf16): the routed and the
// shared gate/up weights (w13), then the routed down weights (w2), each
// 256-byte aligned and the size of its canonical array. The routed down GEMM
// reads them on the packed tiles (gemm_pf.hip, plain epilogue): 4.00 against
// 4.12-4.15 ms for the LDS-staged canonical tiles (prefill shape, no shared
// expert beside it). The shared expert's down GEMM writes fp32 and keeps the
// canonical tiles.
struct PackedLayout {
    size_t w13, sw13, w2, total;
};

PackedLayout packed_layout(const moe_config* c) {
    const size_t El = static_cast<size_t>(c->expert_end - c->expert_begin);
    const size_t H = static_cast<size_t>(c->hidden), I = static_cast<size_t>(c->inter);
    const size_t Is = static_cast<size_t>(c->shared_inter);
    PackedLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align_up(bytes);
        return at;
    };
    L.w13 = take(2 * El * 2 * I * H);
    L.sw13 = take(2 * 2 * Is * H);
    L.w2 = take(2 * El * H * I);
    L.total = off;
    return L;
}

const unsigned char* packed_ptr(const moe_weights* w, size_t off) {
    return w->packed ? static_cast<const unsigned char*>(w->packed) + off : nullptr;
}

template <typename P>
P* at(void* ws, size_t off) {
    return reinterpret_cast<P*>(static_cast<unsigned char*>(ws) + off);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// ---- optional per-stage timing with HIP events (diagnostics only) ------------
// Events are created by moe_profile_enable, never on a call path; while
// enabled, each stage records a start and a stop event on its stream.
struct Profiler {
    bool on = false;
    int cap = 0, n = 0;
    unsigned mask = ~0u;          // stages that record (bit s: stage s)
    std::vector<hipEvent_t> ev;   // 2 per record
    std::vector<int> stage;
} g_prof;

// A record's slot is taken when its start event is recorded, so timers may
// nest. A record whose start event fails is dropped; one whose stop event
// fails is marked with stage -1, which no query counts.
struct StageTimer {
    hipStream_t s;
    int slot = -1;
    StageTimer(int st, hipStream_t str) : s(str) {
        if (!(g_prof.on && g_prof.n < g_prof.cap && ((g_prof.mask >> st) & 1u))) return;
        if (hipEventRecord(g_prof.ev[2 * g_prof.n], s) != hipSuccess) return;
        slot = g_prof.n++;
        g_prof.stage[slot] = st;
    }
    ~StageTimer() {
        if (slot >= 0 && hipEventRecord(g_prof.ev[2 * slot + 1], s) != hipSuccess) g_prof.stage[slot] = -1;
    }
};

int check_ws(const moe_config* c, int64_t T, const void* ws, size_t ws_bytes) {
    if (!ws) return MOE_ERR_INVALID_ARG;
    if (!aligned16(ws)) return MOE_ERR_MISALIGNED;
    if (ws_bytes < layout(c, T).total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return MOE_OK;
}

int64_t capacity_of(const moe_config* c, int64_t T) {
    if (!(c->capacity_factor > 0.0f)) return INT64_MAX;
    return static_cast<int64_t>(ceil(static_cast<double>(c->capacity_factor) * static_cast<double>(T) *
                                     static_cast<double>(c->top_k) / static_cast<double>(c->n_experts)));
}

// ---- stage bodies (arguments already validated) ------------------------------

hipError_t do_router_gemm(const moe_config* c, int64_t T, const void* x, const void* wr, const float* bias,
                          float* logits, void* ws, hipStream_t s) {
    StageTimer tm(MOE_STAGE_ROUTER_GEMM, s);
    const Layout L = layout(c, T);
    GemmArgs g{};
    g.A = g.A_shared = x;
    g.B = g.B_shared = wr;
    g.n_local = 1;
    g.T = static_cast<int>(T);
    g.K = c->hidden;
    g.N = c->n_experts;
    g.C = g.C_shared = logits;
    g.ldc = c->n_experts;
    g.bias = bias;
    g.out_f32 = 1;
    g.partial = at<float>(ws, L.partial);
    // A large bf16 batch: 256 x 256 tiles split along K (a few dozen m-tiles
    // would leave most CUs idle); otherwise the decode tiles' split-K plan.
    if (gemm_elem(c) == Elem::BF16) {
        const GemmPlan pb = plan_router_big(T, c->n_experts, c->hidden);
        if (pb.ksplit > 1) {
            g.ksplit = pb.ksplit;
            hipError_t e = launch_gemm_big(Epi::PLAIN, g, pb, s);
            if (e == hipSuccess) e = launch_splitk_reduce(g, pb.ksplit, s);
            return e;
        }
    }
    const GemmPlan p = plan_dense_splitk(T, c->n_experts, c->hidden, router_chunk(c));
    g.ksplit = p.ksplit;
    hipError_t e = launch_gemm(gemm_elem(c), Epi::PLAIN, g, p, s);
    if (e == hipSuccess) e = launch_splitk_reduce(g, p.ksplit, s);
    return e;
}

hipError_t do_route(const moe_config* c, int64_t T, const float* logits, const float* sbias, int32_t* ids,
                    float* w, hipStream_t s) {
    StageTimer tm(MOE_STAGE_ROUTE, s);
    RouteArgs r{};
    r.logits = logits;
    r.score_bias = sbias;
    r.ids = ids;
    r.w = w;
    r.T = static_cast<int>(T);
    r.E = c->n_experts;
    r.k = c->top_k;
    r.G = c->n_group;
    r.Gk = c->topk_group;
    r.score_fn = c->score_fn;
    r.renorm = c->renormalize;
    r.gamma = c->routed_scale;
    return launch_route(r, s);
}

hipError_t do_dispatch(const moe_config* c, int64_t T, const int32_t* ids, int32_t* raw, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* inv, void* ws, hipStream_t s) {
    StageTimer tm(MOE_STAGE_DISPATCH, s);
    const Layout L = layout(c, T);
    DispatchArgs d{};
    d.ids = ids;
    d.raw = raw;
    d.counts = counts;
    d.offsets = offsets;
    d.perm = perm;
    d.inv = inv;
    d.chunk_hist = at<int32_t>(ws, L.chunk_hist);
    d.chunk_base = at<int32_t>(ws, L.chunk_base);
    d.chunk_bad = at<int32_t>(ws, L.chunk_bad);
    d.bad_ids = at<int32_t>(ws, L.status);
    d.P = T * c->top_k;
    d.E = c->n_experts;
    d.El = c->expert_end - c->expert_begin;
    d.begin = c->expert_begin;
    d.cap = capacity_of(c, T);
    return launch_dispatch(d, s);
}

// Which GEMMs of the shared expert one call launches.
enum class SharedPart { ALL, GATE_UP, DOWN };

// The shared expert's down GEMM when it waits on the side stream for the
// routed gate/up GEMM (shared_down_late): do_routed_ffn launches it right
// after that GEMM and sets `launched` once the join is recorded.
struct SideStream;
struct LateSharedDown {
    SideStream* side;
    const moe_config* c;
    int64_t T;
    const void* x;
    const moe_weights* wt;
    void* shared_out;
    void* ws;
    bool launched;
};
hipError_t launch_late_shared_down(LateSharedDown* d, hipStream_t s);

// Fixed cost of one 256 x 256 item over K, in quarters of the cost of one of
// its 32-row blocks, from per-workgroup timelines of the prefill layer: each
// 64-deep stage of an item of n blocks took f + b n, and the item about o
// outside its K loop, so the fixed part is f / b + o / (b K / 64) blocks.
//   packed gate/up kernel: f 0.28 us, b 0.163 us, o 13 us (K = 7168: 2.4);
//   LDS-staged kernel (both operands through LDS, the down GEMM): f 0.93 us,
//   b 0.104 us, o 10 us (K = 2048: 12).
int item_cost_q(bool packed, int K) {
    const double stages = K / 64.0;
    const double blocks = packed ? 0.28 / 0.163 + 13.0 / (0.163 * stages) : 0.93 / 0.104 + 10.0 / (0.104 * stages);
    return static_cast<int>(4.0 * blocks + 0.5);
}

hipError_t do_routed_ffn(const moe_config* c, int64_t T, const void* x, const int32_t* perm,
                         const int32_t* offsets, const moe_weights* wt, void* rows, void* ws, hipStream_t s,
                         LateSharedDown* late) {
    const Layout L = layout(c, T);
    const Elem el = gemm_elem(c);
    const int El = c->expert_end - c->expert_begin;
    const int64_t H = c->hidden, I = c->inter;
    const int64_t P = T * c->top_k;
    int32_t* sched = at<int32_t>(ws, L.sched);
    hipError_t e;

    // Routed experts: gate/up GEMM with fused SwiGLU, then the down GEMM.
    GemmArgs g1{};
    g1.A = g1.A_shared = x;
    g1.perm = perm;
    g1.gather = 1;
    g1.topk = c->top_k;
    g1.B = g1.B_shared = wt->w13;
    g1.b_stride = 2 * I * H;
    g1.offsets = offsets;
    g1.sched = sched;
    g1.n_local = El;
    g1.T = static_cast<int>(T);
    g1.K = static_cast<int>(H);
    g1.N = static_cast<int>(I);
    g1.inter = static_cast<int>(I);
    g1.C = g1.C_shared = at<void>(ws, L.h);
    g1.ldc = static_cast<int>(I);
    const int64_t per_expert = (P + c->n_experts - 1) / c->n_experts;
    if (quantised(c)) {
        // e4m3 operands: x quantised into the workspace by do_quant_x, h
        // requantised by the gate/up epilogue; FP8 (1x128 fp32 scales, 128x128
        // weight blocks) or MX (E8M0 scales per 32, FP4 weights).
        const bool mx = c->dtype == MOE_DTYPE_MXFP4;
        g1.A = g1.A_shared = at<void>(ws, L.xq);
        g1.A_scale = g1.A_scale_shared = at<void>(ws, L.xs);
        g1.B_scale = g1.B_scale_shared = wt->w13_scale;
        g1.C_scale = g1.C_scale_shared = at<void>(ws, L.hs);
        g1.b_stride = mx ? I * H : 2 * I * H;                  // bytes between experts
        const GemmPlan p1 = plan_quantised(c, Epi::SWIGLU, P, El, per_expert, static_cast<int>(I));
        if ((e = launch_schedule(g1, p1.bm, sched, s)) != hipSuccess) return e;
        {
            StageTimer tm(MOE_STAGE_GATE_UP, s);
            if ((e = launch_quantised(c, Epi::SWIGLU, g1, p1, s)) != hipSuccess) return e;
        }
        if (late && (e = launch_late_shared_down(late, s)) != hipSuccess) return e;
        GemmArgs g2 = g1;
        g2.A = g2.A_shared = at<void>(ws, L.h);
        g2.A_scale = g2.A_scale_shared = at<void>(ws, L.hs);
        g2.perm = nullptr;
        g2.gather = 0;
        g2.B = g2.B_shared = wt->w2;
        g2.B_scale = g2.B_scale_shared = wt->w2_scale;
        g2.b_stride = mx ? H * I / 2 : H * I;
        g2.K = static_cast<int>(I);
        g2.N = static_cast<int>(H);
        g2.inter = 0;
        g2.C = g2.C_shared = rows;
        g2.C_scale = g2.C_scale_shared = nullptr;
        g2.ldc = static_cast<int>(H);
        g2.out_f32 = 0;
        // the down GEMM reuses the gate/up schedule's m-tiles: same row tile
        const GemmPlan p2 = plan_quantised(c, Epi::PLAIN, P, El, per_expert, static_cast<int>(H));
        if (p2.bm != p1.bm) return hipErrorInvalidValue;
        StageTimer tm(MOE_STAGE_DOWN, s);
        return launch_quantised(c, Epi::PLAIN, g2, p2, s);
    }
    GemmPlan p1 = routed_plan(c, Epi::SWIGLU, P, El, per_expert, static_cast<int>(I), wt->packed != nullptr);
    // 256 x 256 tiles read prepacked weights when the caller has them
    const bool pf = p1.big && wt->packed;
    if (pf) {
        p1.big = 2;
        g1.B = g1.B_shared = packed_ptr(wt, packed_layout(c).w13);
    }
    GemmPlan p2 = routed_plan(c, Epi::PLAIN, P, El, per_expert, static_cast<int>(H), wt->packed != nullptr);
    if (p2.bm != p1.bm || p2.big != p1.big) {    // the down GEMM reuses the gate/up schedule's m-tiles
        if (p1.big) {
            p2 = plan_gemm_big(Epi::PLAIN, P, El, static_cast<int>(H));   // the same 256 x 256 m-tiles
        } else {
            p2.big = 0;
            p2.bm = p1.bm;
            p2.nw = p1.nw;
            p2.smajor = p1.smajor;
            p2.n_tiles = (static_cast<int>(H) + 64 * p2.nw - 1) / (64 * p2.nw);
            p2.grid = ((P / p2.bm + El) * p2.n_tiles + 7) / 8 * 8;
        }
    }
    const int4* down_tiles = nullptr;
    if (p1.big) {
        // 256 x 256 tiles: a group's m-tiles have 1..8 blocks of rows, so
        // equal item counts would leave unequal work on the XCDs; both GEMMs
        // get ranges cut by estimated work
        int32_t* ranges = sched + El + 2;
        const XcdSplit sp[2] = {
            {p1.n_tiles, static_cast<int>(p1.grid / 8), item_cost_q(pf, static_cast<int>(H)), ranges},
            {p2.n_tiles, static_cast<int>(p2.grid / 8), item_cost_q(pf, static_cast<int>(I)), ranges + 9}};
        if ((e = launch_schedule(g1, p1.bm, sched, s, sp, 2)) != hipSuccess) return e;
        g1.xcd_range = ranges;
        // each item's tile in a table, so that a workgroup finds it with one
        // load instead of a binary search of dependent loads over the schedule
        // (2.2-2.7 us of every tile's start, measured)
        if (p1.grid + p2.grid <= big_tile_entries(c, T)) {
            int4* const tabs[2] = {at<int4>(ws, L.tiles), at<int4>(ws, L.tiles) + p1.grid};
            const int nt[2] = {p1.n_tiles, p2.n_tiles};
            const int cap[2] = {static_cast<int>(p1.grid), static_cast<int>(p2.grid)};
            if ((e = launch_tile_table(g1, p1.bm, 2, nt, cap, tabs, s)) != hipSuccess) return e;
            g1.tiles = tabs[0];
            down_tiles = tabs[1];
        }
    } else if ((e = launch_schedule(g1, p1.bm, sched, s)) != hipSuccess) {
        return e;
    }
    {
        StageTimer tm(MOE_STAGE_GATE_UP, s);
        if ((e = launch_gemm(el, Epi::SWIGLU, g1, p1, s)) != hipSuccess) return e;
    }
    if (late && (e = launch_late_shared_down(late, s)) != hipSuccess) return e;

    GemmArgs g2 = g1;
    g2.xcd_range = g1.xcd_range ? g1.xcd_range + 9 : nullptr;
    g2.tiles = down_tiles;
    g2.A = g2.A_shared = at<void>(ws, L.h);
    g2.perm = nullptr;
    g2.gather = 0;
    g2.B = g2.B_shared = wt->w2;
    g2.b_stride = H * I;
    g2.K = static_cast<int>(I);
    g2.N = static_cast<int>(H);
    g2.inter = 0;
    g2.C = g2.C_shared = rows;
    g2.ldc = static_cast<int>(H);
    g2.out_f32 = c->dtype == MOE_DTYPE_F32;
    if (pf && p2.big) {                           // the packed tiles, plain epilogue (bf16 rows)
        g2.B = g2.B_shared = packed_ptr(wt, packed_layout(c).w2);
        p2.big = 2;
    }
    StageTimer tm(MOE_STAGE_DOWN, s);
    return launch_gemm(el, Epi::PLAIN, g2, p2, s);
}

bool overlap_shared(const moe_config* c, int64_t T);

// Compute units of the current device (cached per device).
int device_cus() {
    constexpr int kDevices = 64;
    static std::atomic<int> cache[kDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

bool shared_big_tiles(const moe_config* c, int64_t T);

// A bf16 shared expert below 1024 tokens that runs beside the routed
// experts' decode tiles takes the 128 x 128 tiles of gemm_cores.hip, which fit
// on a CU next to a routed workgroup (measured at the full-decode shape, 512
// tokens: 4.03 -> 3.96 ms per layer). From 1024 tokens the 256 x 256 tiles
// stay faster (at the EP8 decode share, 2048 tokens: 0.88 against 0.92 ms),
// since the shared expert's own operand traffic then competes with the
// routed weight stream for the CUs' memory path.
bool shared_cores(const moe_config* c, int64_t T) {
    return c->dtype == MOE_DTYPE_BF16 && !shared_big_tiles(c, T) && overlap_shared(c, T);
}

// The shared expert is one dense group of T rows: from 1024 rows on it is
// compute-bound, and the 256 x 256 LDS-pipelined tiles (bf16, fp8) run it
// faster than the bandwidth-oriented tiles (bf16: 1.4x at T = 2048).
bool shared_big_tiles(const moe_config* c, int64_t T) {
    return (c->dtype == MOE_DTYPE_BF16 || c->dtype == MOE_DTYPE_FP8) && T >= 1024;
}

// Shared expert: every token, a single group (no schedule needed).
hipError_t do_shared_ffn(const moe_config* c, int64_t T, const void* x, const moe_weights* wt, void* shared_out,
                         void* ws, hipStream_t s, SharedPart part = SharedPart::ALL) {
    const bool gate_up = part != SharedPart::DOWN;
    const Layout L = layout(c, T);
    const Elem el = gemm_elem(c);
    const int64_t H = c->hidden, Is = c->shared_inter;
    hipError_t e;
    GemmArgs s1{};
    s1.A = s1.A_shared = x;
    s1.B = s1.B_shared = wt->shared_w13;
    s1.n_local = 0;
    s1.has_shared = 1;
    s1.T = static_cast<int>(T);
    s1.K = static_cast<int>(H);
    s1.N = static_cast<int>(Is);
    s1.inter = static_cast<int>(Is);
    s1.C = s1.C_shared = at<void>(ws, L.h_shared);
    s1.ldc = static_cast<int>(Is);
    if (quantised(c)) {
        s1.A = s1.A_shared = at<void>(ws, L.xq);
        s1.A_scale = s1.A_scale_shared = at<void>(ws, L.xs);
        s1.B_scale = s1.B_scale_shared = wt->shared_w13_scale;
        s1.C_scale = s1.C_scale_shared = at<void>(ws, L.hs_shared);
        const bool bigq = c->dtype == MOE_DTYPE_FP8 && shared_big_tiles(c, T);
        const GemmPlan q1 = bigq ? plan_gemm_fp8_big(Epi::SWIGLU, T, 1, static_cast<int>(Is))
                                 : plan_quantised(c, Epi::SWIGLU, T, 1, T, static_cast<int>(Is));
        if (gate_up) {
            StageTimer tm(MOE_STAGE_SHARED_GATE_UP, s);
            if ((e = launch_quantised(c, Epi::SWIGLU, s1, q1, s)) != hipSuccess) return e;
        }
        if (part == SharedPart::GATE_UP) return hipSuccess;
        GemmArgs s2 = s1;
        s2.A = s2.A_shared = at<void>(ws, L.h_shared);
        s2.A_scale = s2.A_scale_shared = at<void>(ws, L.hs_shared);
        s2.B = s2.B_shared = wt->shared_w2;
        s2.B_scale = s2.B_scale_shared = wt->shared_w2_scale;
        s2.K = static_cast<int>(Is);
        s2.N = static_cast<int>(H);
        s2.inter = 0;
        s2.C = s2.C_shared = shared_out;
        s2.C_scale = s2.C_scale_shared = nullptr;
        s2.ldc = static_cast<int>(H);
        s2.out_f32 = 1;
        const GemmPlan q2 = bigq ? plan_gemm_fp8_big(Epi::PLAIN, T, 1, static_cast<int>(H))
                                 : plan_quantised(c, Epi::PLAIN, T, 1, T, static_cast<int>(H));
        StageTimer tm(MOE_STAGE_SHARED_DOWN, s);
        return launch_quantised(c, Epi::PLAIN, s2, q2, s);
    }
    if (shared_cores(c, T)) {
        const GemmPlan q1 = plan_gemm_cores(Epi::SWIGLU, T, static_cast<int>(Is), device_cus());
        if (gate_up) {
            StageTimer tm(MOE_STAGE_SHARED_GATE_UP, s);
            if ((e = launch_gemm_cores(Epi::SWIGLU, s1, q1, s)) != hipSuccess) return e;
        }
        if (part == SharedPart::GATE_UP) return hipSuccess;
        GemmArgs s2 = s1;
        s2.A = s2.A_shared = at<void>(ws, L.h_shared);
        s2.B = s2.B_shared = wt->shared_w2;
        s2.K = static_cast<int>(Is);
        s2.N = static_cast<int>(H);
        s2.inter = 0;
        s2.C = s2.C_shared = shared_out;
        s2.ldc = static_cast<int>(H);
        s2.out_f32 = 1;
        const GemmPlan q2 = plan_gemm_cores(Epi::PLAIN, T, static_cast<int>(H), device_cus());
        StageTimer tm(MOE_STAGE_SHARED_DOWN, s);
        return launch_gemm_cores(Epi::PLAIN, s2, q2, s);
    }
    const bool big = shared_big_tiles(c, T);
    // 256 x 256 tiles read prepacked weights when the caller has them
    const bool pf = big && c->dtype == MOE_DTYPE_BF16 && wt->packed;
    if (pf) s1.B = s1.B_shared = packed_ptr(wt, packed_layout(c).sw13);
    const GemmPlan q1 = pf    ? plan_gemm_pf(T, 1, static_cast<int>(Is))
                        : big ? plan_gemm_big(Epi::SWIGLU, T, 1, static_cast<int>(Is))
                              : plan_gemm(el, Epi::SWIGLU, T, 1, T, static_cast<int>(Is));
    if (gate_up) {
        StageTimer tm(MOE_STAGE_SHARED_GATE_UP, s);
        if ((e = launch_gemm(el, Epi::SWIGLU, s1, q1, s)) != hipSuccess) return e;
    }
    if (part == SharedPart::GATE_UP) return hipSuccess;
    GemmArgs s2 = s1;
    s2.A = s2.A_shared = at<void>(ws, L.h_shared);
    s2.B = s2.B_shared = wt->shared_w2;
    s2.K = static_cast<int>(Is);
    s2.N = static_cast<int>(H);
    s2.inter = 0;
    s2.C = s2.C_shared = shared_out;
    s2.ldc = static_cast<int>(H);
    s2.out_f32 = 1;          // the shared output stays fp32 (it is never exchanged)
    const GemmPlan q2 = big ? plan_gemm_big(Epi::PLAIN, T, 1, static_cast<int>(H))
                            : plan_gemm(el, Epi::PLAIN, T, 1, T, static_cast<int>(H));
    StageTimer tm(MOE_STAGE_SHARED_DOWN, s);
    return launch_gemm(el, Epi::PLAIN, s2, q2, s);
}

// The shared expert runs on a second stream of the same device, concurrently
// with the routed path (NVIDIA "Optimizing DeepSeek R1 throughput on
// Blackwell", section "Multi-stream": shared and routed experts on two
// streams; Perplexity, "Overlapping compute and communication": the shared
// expert fills the dispatch gap). The stream and its two events are created
// on first use on a device and kept until the process ends.
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, mid = nullptr, join = nullptr;
};
std::mutex g_side_mu;
std::unordered_map<int, SideStream> g_side;

hipError_t side_stream(SideStream** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    SideStream& ss = g_side[dev];
    if (!ss.stream) {
        if ((e = hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&ss.mid, hipEventDisableTiming)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming)) != hipSuccess) return e;
    }
    *out = &ss;
    return hipSuccess;
}

// Launches the shared expert on the side stream, ordered after everything
// already on `s`; the caller joins with join_shared before reading shared_out.
// With `late_down` only its gate/up GEMM is launched here: the caller passes
// a LateSharedDown to do_routed_ffn, which launches the down GEMM (and
// records the join) once the routed gate/up GEMM is on `s`.
hipError_t fork_shared(const moe_config* c, int64_t T, const void* x, const moe_weights* wt, void* shared_out,
                       void* ws, hipStream_t s, bool late_down, SideStream** side) {
    hipError_t e = side_stream(side);
    if (e != hipSuccess) return e;
    SideStream* ss = *side;
    if ((e = hipEventRecord(ss->fork, s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(ss->stream, ss->fork, 0)) != hipSuccess) return e;
    const SharedPart part = late_down ? SharedPart::GATE_UP : SharedPart::ALL;
    e = do_shared_ffn(c, T, x, wt, shared_out, ws, ss->stream, part);
    if (late_down && e == hipSuccess) return hipSuccess;       // the join follows the late down GEMM
    // the join also follows whatever was enqueued before an error
    const hipError_t j = hipEventRecord(ss->join, ss->stream);
    return e != hipSuccess ? e : j;
}

hipError_t launch_late_shared_down(LateSharedDown* d, hipStream_t s) {
    SideStream* ss = d->side;
    hipError_t e = hipEventRecord(ss->mid, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(ss->stream, ss->mid, 0);
    if (e == hipSuccess) e = do_shared_ffn(d->c, d->T, d->x, d->wt, d->shared_out, d->ws, ss->stream, SharedPart::DOWN);
    // the join follows whatever was enqueued on the side stream, also after an error
    const hipError_t j = hipEventRecord(ss->join, ss->stream);
    if (j == hipSuccess) d->launched = true;
    return e != hipSuccess ? e : j;
}

// After a late fork whose join was never recorded (an error before the
// routed gate/up GEMM), the join still has to follow the shared gate/up.
hipError_t close_late_fork(const LateSharedDown& d) {
    return d.launched ? hipSuccess : hipEventRecord(d.side->join, d.side->stream);
}

hipError_t join_shared(SideStream* ss, hipStream_t s) { return hipStreamWaitEvent(s, ss->join, 0); }

// The shared expert runs beside the routed experts whenever there is one.
// With bandwidth-bound routed tiles it fills their idle matrix cores (the EP8
// decode layer and the capacity-limited fp8 layer run about 20% and 4.5%
// faster overlapped). At prefill both take the 256 x 256 tiles, which hold a
// whole CU each, so the two only take turns on the CUs; what overlap still
// gains there is the routed GEMMs' tails (the bf16 prefill layer 13.28 ->
// 13.14 ms per step).
bool overlap_shared(const moe_config* c, int64_t) { return c->shared_inter > 0; }

// A shared expert that runs beside the routed experts launches its down GEMM
// only once the routed gate/up GEMM has finished, so that it runs beside the
// routed down GEMM. That GEMM's workgroups need not fill a whole number of
// rounds on the CUs (the EP8 decode share: 448 workgroups of one per CU), and
// the routed gate/up GEMM, which streams twice the weight bytes, keeps more
// of the GPU. Measured per layer: EP8 decode share 0.897 -> 0.884 ms, FP4
// full decode 1.254 -> 1.245 ms, bf16 full decode 3.962 -> 3.951 ms, the
// capacity-limited fp8 layer unchanged.
bool shared_down_late(const moe_config* c, int64_t T) { return overlap_shared(c, T); }

// FP8 / MXFP4: x -> e4m3 codes + per-(row, 128 or 32 columns) scales in the
// workspace, read by both the routed and the shared gate/up GEMMs.
hipError_t do_quant_x(const moe_config* c, int64_t T, const void* x, void* ws, hipStream_t s) {
    if (!quantised(c)) return hipSuccess;
    const Layout L = layout(c, T);
    StageTimer tm(MOE_STAGE_QUANT, s);
    if (c->dtype == MOE_DTYPE_MXFP4)
        return launch_quant_mx(x, at<uint8_t>(ws, L.xq), at<uint8_t>(ws, L.xs), T, c->hidden, s);
    return launch_quant_fp8(x, at<uint8_t>(ws, L.xq), at<float>(ws, L.xs), T, c->hidden, s);
}

hipError_t do_expert_ffn(const moe_config* c, int64_t T, const void* x, const int32_t* perm,
                         const int32_t* offsets, const moe_weights* wt, void* rows, void* shared_out, void* ws,
                         hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_side_mu);
    SideStream* side = nullptr;
    hipError_t e = do_quant_x(c, T, x, ws, s);
    if (e != hipSuccess) return e;
    const bool late = shared_down_late(c, T);
    if (overlap_shared(c, T)) e = fork_shared(c, T, x, wt, shared_out, ws, s, late, &side);
    LateSharedDown ld{side, c, T, x, wt, shared_out, ws, false};
    if (e == hipSuccess) e = do_routed_ffn(c, T, x, perm, offsets, wt, rows, ws, s, side && late ? &ld : nullptr);
    if (side) {                                                // always rejoin the side stream
        hipError_t j = late ? close_late_fork(ld) : hipSuccess;
        if (j == hipSuccess) j = join_shared(side, s);
        if (e == hipSuccess) e = j;
    } else if (e == hipSuccess && c->shared_inter > 0) {
        e = do_shared_ffn(c, T, x, wt, shared_out, ws, s);
    }
    return e;
}

hipError_t do_combine(const moe_config* c, int64_t T, const void* rows, const int32_t* inv, const float* w,
                      const void* shared_out, void* y, hipStream_t s) {
    StageTimer tm(MOE_STAGE_COMBINE, s);
    CombineArgs a{};
    a.rows = rows;
    a.inv = inv;
    a.w = w;
    a.shared = static_cast<const float*>(shared_out);
    a.y = y;
    a.T = T;
    a.H = c->hidden;
    a.k = c->top_k;
    a.rows_f32 = c->dtype == MOE_DTYPE_F32;
    a.out_f32 = c->out_dtype == MOE_DTYPE_F32;
    return launch_combine(a, s);
}

bool weights_ok(const moe_config* c, const moe_weights* w) {
    if (!w || !w->w13 || !w->w2) return false;
    if (w->packed && (c->dtype != MOE_DTYPE_BF16 || !aligned16(w->packed))) return false;
    if (!aligned16(w->w13) || !aligned16(w->w2)) return false;
    if (c->shared_inter > 0 && (!w->shared_w13 || !w->shared_w2 || !aligned16(w->shared_w13) ||
                                !aligned16(w->shared_w2)))
        return false;
    if (quantised(c)) {
        if (!w->w13_scale || !w->w2_scale) return false;
        if (c->shared_inter > 0 && (!w->shared_w13_scale || !w->shared_w2_scale)) return false;
        // MX scale rows are read 8 bytes at a time
        auto al8 = [](const void* p) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % 8 == 0; };
        if (!al8(w->w13_scale) || !al8(w->w2_scale) || !al8(w->shared_w13_scale) || !al8(w->shared_w2_scale))
            return false;
    }
    return true;
}

// ---- the whole layer -----------------------------------------------------------

// Argument checks of moe_forward and moe_forward_noalloc (the workspace aside).
int check_forward(const moe_config* cfg, int64_t T, const void* x, const void* w_router, const moe_weights* weights,
                  const void* y, const float* logits_out, const int32_t* topk_ids_out) {
    int st = validate(cfg);
    if (st) return st;
    if (T < 0 || T > INT32_MAX / 16) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !y || !weights_ok(cfg, weights)) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(y) || (logits_out && !aligned16(logits_out)) ||
        (topk_ids_out && !aligned16(topk_ids_out)))
        return MOE_ERR_MISALIGNED;
    if (!offsets_fit(cfg, T, false)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// Router GEMM, route, dispatch, experts, combine on `stream`, with workspace
// `ws` (already checked). With `side_ok` the shared expert runs beside the
// routed path on the side stream where that pays (overlap_shared); without
// it, on `stream` after the routed experts, with the same kernels.
int forward_body(const moe_config* cfg, int64_t T, const void* x, const void* w_router, const float* router_bias,
                 const float* score_bias, const moe_weights* weights, void* y, float* logits_out,
                 int32_t* topk_ids_out, void* ws, hipStream_t stream, bool side_ok) {
    const Layout L = layout(cfg, T);
    float* logits = logits_out ? logits_out : at<float>(ws, L.logits);
    int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, L.ids);
    float* w = at<float>(ws, L.w);
    int32_t* offsets = at<int32_t>(ws, L.offsets);
    int32_t* perm = at<int32_t>(ws, L.perm);
    int32_t* inv = at<int32_t>(ws, L.inv);
    void* rows = at<void>(ws, L.rows);
    void* shared_out = cfg->shared_inter > 0 ? at<void>(ws, L.shared_out) : nullptr;
    // At decode shapes the shared expert (which needs only x) starts first,
    // on the side stream, and runs beside the routing kernels and the routed
    // experts' grouped GEMMs (measured on the EP8 decode share: 0.917 ->
    // 0.892 ms per layer).
    std::lock_guard<std::mutex> lk(g_side_mu);
    SideStream* side = nullptr;
    const bool overlap = side_ok && overlap_shared(cfg, T);
    const bool late = shared_down_late(cfg, T);
    hipError_t e = do_quant_x(cfg, T, x, ws, stream);
    if (e == hipSuccess && overlap) e = fork_shared(cfg, T, x, weights, shared_out, ws, stream, late, &side);
    LateSharedDown ld{side, cfg, T, x, weights, shared_out, ws, false};
    if (e == hipSuccess) e = do_router_gemm(cfg, T, x, w_router, router_bias, logits, ws, stream);
    if (e == hipSuccess) e = do_route(cfg, T, logits, score_bias, ids, w, stream);
    if (e == hipSuccess)
        e = do_dispatch(cfg, T, ids, at<int32_t>(ws, L.raw), at<int32_t>(ws, L.counts), offsets, perm, inv, ws,
                        stream);
    if (e == hipSuccess)
        e = do_routed_ffn(cfg, T, x, perm, offsets, weights, rows, ws, stream, side && late ? &ld : nullptr);
    if (side) {
        // always rejoin the side stream
        hipError_t j = late ? close_late_fork(ld) : hipSuccess;
        if (j == hipSuccess) j = join_shared(side, stream);
        if (e == hipSuccess) e = j;
    } else if (e == hipSuccess && shared_out) {
        e = do_shared_ffn(cfg, T, x, weights, shared_out, ws, stream);
    }
    if (e == hipSuccess) e = do_combine(cfg, T, rows, inv, w, shared_out, y, stream);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ---- the workspace of moe_forward_noalloc ---------------------------------------
// A device array of the library's own, one copy per GPU, held until the
// process ends. In host code `scratch` names a host-side stand-in, not the
// device memory: its device address is looked up once per device (with that
// device current) by hipGetSymbolAddress, and only that address is ever
// passed on. The layer writes every workspace region before reading it, so
// nothing in it has to start at zero.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];

hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MOE_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
        case MOE_ERR_HIP: return "HIP launch error";
        case MOE_ERR_ABI_MISMATCH: return "ABI version mismatch";
        default: return "unknown status";
    }
}

int moe_validate_config(const moe_config* cfg) { return validate(cfg); }

int moe_workspace_bytes(const moe_config* cfg, int64_t max_tokens, size_t* bytes) {
    int st = validate(cfg);
    if (st) return st;
    if (max_tokens < 0 || !bytes) return MOE_ERR_INVALID_ARG;
    *bytes = layout(cfg, max_tokens).total;
    return MOE_OK;
}

int moe_packed_weights_bytes(const moe_config* cfg, size_t* bytes) {
    int st = validate(cfg);
    if (st) return st;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    if (cfg->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
    *bytes = packed_layout(cfg).total;
    return MOE_OK;
}

int moe_prepack_weights(const moe_config* cfg, const moe_weights* canonical, void* packed, size_t packed_bytes,
                        hipStream_t stream) {
    int st = validate(cfg);
    if (st) return st;
    if (cfg->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
    const moe_weights* w = canonical;
    if (!w || !w->w13 || !w->w2 || !packed) return MOE_ERR_INVALID_ARG;
    if (cfg->shared_inter > 0 && !w->shared_w13) return MOE_ERR_INVALID_ARG;
    if (!aligned16(w->w13) || !aligned16(w->w2) || (reinterpret_cast<uintptr_t>(packed) % kAlign) ||
        (cfg->shared_inter > 0 && !aligned16(w->shared_w13)))
        return MOE_ERR_MISALIGNED;
    const PackedLayout L = packed_layout(cfg);
    if (packed_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    unsigned char* d = static_cast<unsigned char*>(packed);
    const int El = cfg->expert_end - cfg->expert_begin, H = cfg->hidden, I = cfg->inter, Is = cfg->shared_inter;
    hipError_t e = launch_prepack(w->w13, d + L.w13, El, I, H, stream);
    if (e == hipSuccess && Is > 0) e = launch_prepack(w->shared_w13, d + L.sw13, 1, Is, H, stream);
    if (e == hipSuccess) e = launch_prepack_down(w->w2, d + L.w2, El, H, I, stream);
    return hip_status(e);
}

int moe_router_gemm(const moe_config* cfg, int64_t T, const void* x, const void* w_router, const float* router_bias,
                    float* logits, void* ws, size_t ws_bytes, hipStream_t stream) {
    int st = validate(cfg);
    if (st) return st;
    if (T < 0 || T > INT32_MAX / 16) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !logits) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(logits)) return MOE_ERR_MISALIGNED;
    if (!offsets_fit(cfg, T, true)) return MOE_ERR_UNSUPPORTED;
    if ((st = check_ws(cfg, T, ws, ws_bytes))) return st;
    return hip_status(do_router_gemm(cfg, T, x, w_router, router_bias, logits, ws, stream));
}

int moe_route(const moe_config* cfg, int64_t T, const float* logits, const float* score_bias, int32_t* topk_ids,
              float* topk_w, hipStream_t stream) {
    int st = validate(cfg);
    if (st) return st;
    if (T < 0 || T > INT32_MAX / 16) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
    if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w)) return MOE_ERR_MISALIGNED;
    return hip_status(do_route(cfg, T, logits, score_bias, topk_ids, topk_w, stream));
}

int moe_dispatch(const moe_config* cfg, int64_t T, const int32_t* topk_ids, int32_t* raw_counts, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* inv, void* ws, size_t ws_bytes, hipStream_t stream) {
    int st = validate(cfg);
    if (st) return st;
    if (T < 0 || T > INT32_MAX / 16) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!topk_ids || !counts || !offsets || !perm || !inv) return MOE_ERR_INVALID_ARG;
    if (!aligned16(topk_ids) || !aligned16(counts) || !aligned16(offsets) || !aligned16(perm) || !aligned16(inv) ||
        (raw_counts && !aligned16(raw_counts)))
        return MOE_ERR_MISALIGNED;
    if ((st = check_ws(cfg, T, ws, ws_bytes))) return st;
    return hip_status(do_dispatch(cfg, T, topk_ids, raw_counts, counts, offsets, perm, inv, ws, stream));
}

int moe_expert_ffn(const moe_config* cfg, int64_t T, const void* x, const int32_t* perm, const int32_t* offsets,
                   const moe_weights* weights, void* out_rows, void* shared_out, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
    int st = validate(cfg);
    if (st) return st;
    if (T < 0 || T > INT32_MAX / 16) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !perm || !offsets || !out_rows || !weights_ok(cfg, weights)) return MOE_ERR_INVALID_ARG;
    if (cfg->shared_inter > 0 && !shared_out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(perm) || !aligned16(offsets) || !aligned16(out_rows) ||
        (shared_out && !aligned16(shared_out)))
        return MOE_ERR_MISALIGNED;
    if (!offsets_fit(cfg, T, false)) return MOE_ERR_UNSUPPORTED;
    if ((st = check_ws(cfg, T, ws, ws_bytes))) return st;
    return hip_status(do_expert_ffn(cfg, T, x, perm, offsets, weights, out_rows, shared_out, ws, stream));
}

int moe_combine(const moe_config* cfg, int64_t T, const void* out_rows, const int32_t* inv, const float* topk_w,
                const void* shared_out, void* y, hipStream_t stream) {
    int st = validate(cfg);
    if (st) return st;
    if (T < 0 || T > INT32_MAX / 16) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!out_rows || !inv || !topk_w || !y) return MOE_ERR_INVALID_ARG;
    if (!aligned16(out_rows) || !aligned16(inv) || !aligned16(topk_w) || !aligned16(y) ||
        (shared_out && !aligned16(shared_out)))
        return MOE_ERR_MISALIGNED;
    return hip_status(do_combine(cfg, T, out_rows, inv, topk_w, shared_out, y, stream));
}

int moe_forward(const moe_config* cfg, int64_t T, const void* x, const void* w_router, const float* router_bias,
                const float* score_bias, const moe_weights* weights, void* y, float* logits_out,
                int32_t* topk_ids_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_forward(cfg, T, x, w_router, weights, y, logits_out, topk_ids_out);
    if (st || T == 0) return st;
    if ((st = check_ws(cfg, T, ws, ws_bytes))) return st;
    return forward_body(cfg, T, x, w_router, router_bias, score_bias, weights, y, logits_out, topk_ids_out, ws,
                        stream, true);
}

int moe_forward_noalloc(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                        const float* router_bias, const float* score_bias, const moe_weights* weights, void* y,
                        float* logits_out, int32_t* topk_ids_out, hipStream_t stream) {
    int st = check_forward(cfg, T, x, w_router, weights, y, logits_out, topk_ids_out);
    if (st || T == 0) return st;
    if (layout(cfg, T).total > kScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return MOE_ERR_HIP;
    // the shared expert runs on `stream` itself: no side stream or event is
    // created (the kernels are those moe_forward picks, so results are equal)
    return forward_body(cfg, T, x, w_router, router_bias, score_bias, weights, y, logits_out, topk_ids_out, ws,
                        stream, false);
}

int moe_dispatch_errors(const void* ws, size_t ws_bytes, hipStream_t stream, int64_t* bad_ids) {
    if (!bad_ids) return MOE_ERR_INVALID_ARG;
    const void* src = ws;
    if (!ws) {
        void* p = nullptr;                   // the moe_forward_noalloc array of the current device
        if (scratch_address(&p) != hipSuccess) return MOE_ERR_HIP;
        src = p;
    } else {
        if (!aligned16(ws)) return MOE_ERR_MISALIGNED;
        if (ws_bytes < kStatusBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
    }
    int32_t word = 0;
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipMemcpy(&word, src, sizeof(word), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return MOE_ERR_HIP;
    *bad_ids = word;
    return MOE_OK;
}

int moe_quantize_fp8(const moe_config* cfg, int64_t rows, const void* x, uint8_t* q, float* scale,
                     hipStream_t stream) {
    int st = validate(cfg);
    if (st) return st;
    if (rows < 0 || rows > INT32_MAX) return MOE_ERR_INVALID_ARG;
    if (rows == 0) return MOE_OK;
    if (!x || !q || !scale) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(q) || !aligned16(scale)) return MOE_ERR_MISALIGNED;
    return hip_status(launch_quant_fp8(x, q, scale, rows, cfg->hidden, stream));
}

int moe_quantize_mx(const moe_config* cfg, int64_t rows, const void* x, uint8_t* q, uint8_t* scale,
                    hipStream_t stream) {
    int st = validate(cfg);
    if (st) return st;
    if (cfg->dtype != MOE_DTYPE_MXFP4) return MOE_ERR_INVALID_ARG;
    if (rows < 0 || rows > INT32_MAX) return MOE_ERR_INVALID_ARG;
    if (rows == 0) return MOE_OK;
    if (!x || !q || !scale) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(q)) return MOE_ERR_MISALIGNED;
    return hip_status(launch_quant_mx(x, q, scale, rows, cfg->hidden, stream));
}

int moe_expert_load(const moe_config* cfg, int64_t T, const int32_t* topk_ids, int64_t* load, hipStream_t stream) {
    int st = validate(cfg);
    if (st) return st;
    if (T < 0) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!topk_ids || !load) return MOE_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(load) % 8) return MOE_ERR_MISALIGNED;
    return hip_status(launch_expert_load(topk_ids, T * cfg->top_k, cfg->n_experts, load, stream));
}

int moe_eplb_plan(const int64_t* load, int n_experts, int n_ranks, int n_redundant, int32_t* replicas,
                  int32_t* slot_expert, double* rank_load, double* imbalance) {
    if (!load || !replicas || !slot_expert || !rank_load || !imbalance) return MOE_ERR_INVALID_ARG;
    if (n_experts <= 0 || n_ranks <= 0 || n_redundant < 0) return MOE_ERR_INVALID_ARG;
    if ((static_cast<int64_t>(n_experts) + n_redundant) % n_ranks != 0) return MOE_ERR_INVALID_ARG;
    for (int e = 0; e < n_experts; ++e)
        if (load[e] < 0) return MOE_ERR_INVALID_ARG;
    plan_placement(load, n_experts, n_ranks, n_redundant, replicas, slot_expert, rank_load);
    double mx = rank_load[0], sum = 0.0;
    for (int g = 0; g < n_ranks; ++g) {
        mx = rank_load[g] > mx ? rank_load[g] : mx;
        sum += rank_load[g];
    }
    *imbalance = sum > 0.0 ? mx / (sum / n_ranks) : 1.0;
    return MOE_OK;
}

int moe_profile_enable(int max_records) {
    if (max_records < 0) return MOE_ERR_INVALID_ARG;
    const unsigned mask = g_prof.mask;          // the stage selection survives
    for (hipEvent_t e : g_prof.ev)
        if (e) (void)hipEventDestroy(e);
    g_prof = Profiler{};
    g_prof.mask = mask;
    if (max_records == 0) return MOE_OK;
    g_prof.ev.resize(2 * static_cast<size_t>(max_records));
    g_prof.stage.resize(max_records);
    for (auto& e : g_prof.ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            e = nullptr;
            return MOE_ERR_HIP;        // left disabled; the next call destroys what was created
        }
    }
    g_prof.cap = max_records;
    g_prof.on = true;
    return MOE_OK;
}

int moe_profile_reset(void) {
    g_prof.n = 0;
    return MOE_OK;
}

int moe_profile_select(unsigned stage_mask) {
    g_prof.mask = stage_mask;
    return MOE_OK;
}

int moe_profile_query(int stage, double* total_ms, int* count) {
    if (!total_ms || !count || stage < 0 || stage >= MOE_STAGE_COUNT) return MOE_ERR_INVALID_ARG;
    double tot = 0.0;
    int cnt = 0;
    for (int i = 0; i < g_prof.n; ++i) {
        if (g_prof.stage[i] != stage) continue;
        if (hipEventSynchronize(g_prof.ev[2 * i + 1]) != hipSuccess) return MOE_ERR_HIP;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess) return MOE_ERR_HIP;
        tot += ms;
        ++cnt;
    }
    *total_ms = tot;
    *count = cnt;
    return MOE_OK;
}

int moe_mfma_loop(int64_t iters, uint64_t* out, double* flops, hipStream_t stream) {
    if (iters < 1 || iters > (int64_t{1} << 40) || !out || !flops) return MOE_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(out) % 8) return MOE_ERR_MISALIGNED;
    return hip_status(launch_mfma_loop(iters, reinterpret_cast<unsigned long long*>(out), flops, stream));
}

int moe_stream_read(const void* src, int64_t bytes, uint32_t* out, hipStream_t stream) {
    if (bytes < 0 || bytes % 16 || (bytes > 0 && !src) || !out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(src) || reinterpret_cast<uintptr_t>(out) % 4) return MOE_ERR_MISALIGNED;
    if (bytes == 0) return MOE_OK;
    return hip_status(launch_stream_read(src, bytes, out, stream));
}

}  // extern "C"
