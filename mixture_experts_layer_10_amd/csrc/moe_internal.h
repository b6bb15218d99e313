// Internal interface between the C ABI (moe_api.cpp) and the kernel
// translation units. Host-side launch functions; each returns a hipError_t.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Element formats of the grouped GEMM operands.
enum class Elem : int { F32 = 0, BF16 = 1, FP8 = 2 };

// --- router (K2) -------------------------------------------------------------
struct RouteArgs {
    const float* logits;      // [T, E]
    const float* score_bias;  // [E] or null
    int32_t* ids;             // [T, k]
    float* w;                 // [T, k]
    int T, E, k, G, Gk, score_fn, renorm;
    float gamma;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s);

// --- dispatch (K3) -----------------------------------------------------------
struct DispatchArgs {
    const int32_t* ids;       // [P]
    int32_t* raw;             // [El] or null
    int32_t* counts;          // [El]
    int32_t* offsets;         // [El + 1]
    int32_t* perm;            // [P]
    int32_t* inv;             // [P]
    int32_t* chunk_hist;      // [nchunk, El] scratch
    int32_t* chunk_base;      // [nchunk, El] scratch
    int32_t* chunk_bad;       // [nchunk] scratch: ids outside [0, E) per chunk
    int32_t* bad_ids;         // [1]: their total over the batch (the error word)
    int64_t P;                // T * k
    int E, El, begin;
    int64_t cap;              // capacity, or INT64_MAX
};
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);
// Pairs per histogram/scatter block: small batches take short blocks, so that
// more workgroups share the work and each makes fewer passes; large batches
// long ones, so that the per-block histograms stay few. A function of P
// only, so the workspace layout and the kernels agree.
__host__ __device__ inline int64_t dispatch_chunk(int64_t P) { return P <= 16384 ? 512 : 2048; }
inline int64_t dispatch_chunks(int64_t P) { return (P + dispatch_chunk(P) - 1) / dispatch_chunk(P); }
// The most blocks any batch of at most P pairs uses (the short blocks end at
// 16384 pairs), so that a workspace sized for P serves every smaller batch.
inline int64_t dispatch_chunks_upto(int64_t P) {
    const int64_t a = dispatch_chunks(P), b = dispatch_chunks(P < 16384 ? P : 16384);
    return a > b ? a : b;
}

// --- grouped GEMM (K1, K5, K6) ----------------------------------------------
enum class Epi : int { SWIGLU = 0, PLAIN = 1 };

struct GemmArgs {
    // A operand: routed rows (gathered through perm when gather != 0) and
    // shared-expert rows (token t = row).
    const void* A;            // routed-row source
    const void* A_shared;     // shared-row source (may equal A)
    const void* A_scale;      // FP8: float [rows, K/128]; MXFP4: E8M0 bytes [rows, K/32]
    const void* A_scale_shared;
    const int32_t* perm;      // gather: token = perm[row] / topk
    int gather;
    int topk;
    // B operand: [n_local, N_B, K] routed weights, [N_B, K] shared weights.
    const void* B;
    const void* B_shared;
    const void* B_scale;      // FP8: float [n_local, N_B/128, K/128]; MXFP4: bytes [n_local, N_B, K/32]
    const void* B_scale_shared;
    int64_t b_stride;         // elements between routed experts (MXFP4: bytes)
    // Groups: rows of routed group g are offsets[g] .. offsets[g+1]-1;
    // group n_local (if has_shared) has T rows.
    const int32_t* offsets;   // [n_local + 1], or null for a single dense group
    const int32_t* sched;     // [n_groups + 1] m-tile prefix
    // Optional [9]: the launch's items dealt to the 8 XCDs by estimated work,
    // XCD x taking items xcd_range[x] .. xcd_range[x+1]-1 (schedule_kernel);
    // null: equal item counts per XCD.
    const int32_t* xcd_range;
    // Optional: the launch's items as tiles, tiles[L] = {g | nt << 16, row0,
    // m0, rows} (launch_tile_table); null: found from the schedule.
    const int4* tiles;
    int n_local, has_shared, T;
    int K;                    // reduction length
    int N;                    // output columns (I for SWIGLU, else N_B)
    int inter;                // SWIGLU: row offset of the up projection in B
    // Outputs
    void* C;                  // routed rows [rows, ldc]
    void* C_shared;           // shared rows [T, ldc]
    void* C_scale;            // SWIGLU, FP8: float [rows, N/128]; MXFP4: E8M0 bytes [rows, N/32]
    void* C_scale_shared;
    int ldc;
    const float* bias;        // PLAIN fp32 out: per-column bias or null
    int out_f32;              // PLAIN: 1 -> fp32 output, 0 -> bf16 output
    // Split-K (PLAIN, fp32 output, single group only): K-slice s of tile t
    // writes fp32 partial sums to partial[s][row][col]; a reduce kernel adds
    // the slices and the bias into C.
    int ksplit;               // >= 1
    float* partial;           // [ksplit, T, ldc] when ksplit > 1
};

struct GemmPlan {
    int bm;                   // rows per tile
    int nw;                   // wavefronts per workgroup (4 or 8)
    int smajor;               // weights consumed sub-run by sub-run (one register buffer)
    int big;                  // 256 x 256 tiles: 1 LDS-pipelined (gemm_big.hip), 2 on packed weights (gemm_pf.hip)
    int n_tiles;              // column tiles per group
    int ksplit;               // K slices per tile
    int64_t grid;             // workgroups launched (upper bound on tiles * ksplit)
};
GemmPlan plan_gemm(Elem e, Epi epi, int64_t rows_upper, int n_groups, int64_t expected_rows_per_group, int N);
// The m-tile schedule of a grouped GEMM: sched[g] = m-tiles of the groups
// before g (row tiles of bm rows). Each XcdSplit also gets, for one launch of
// 256 x 256 tiles on that schedule (balanced row split), the item ranges of
// the 8 XCDs, cut where the estimated work (32-row blocks of an item plus
// cost_q / 4 blocks of fixed cost per item) reaches x / 8 of the total, each
// range at most `cap` items (the launch's workgroup slots per XCD, grid / 8,
// so that every item has a workgroup).
struct XcdSplit {
    int n_tiles;              // column tiles per m-tile
    int cap;                  // grid / 8
    int cost_q;               // fixed cost per item, in quarter blocks
    int32_t* out;             // [9] item boundaries
};
hipError_t launch_schedule(const GemmArgs& a, int bm, int32_t* sched, hipStream_t s, const XcdSplit* splits = nullptr,
                           int n_splits = 0);
// Writes the items of up to two launches on a's schedule (row tiles of bm
// rows, balanced split, n_tiles[i] column tiles, at most cap[i] items) as
// tiles: tables[i][L] = {g | nt << 16, row0, m0, rows}.
hipError_t launch_tile_table(const GemmArgs& a, int bm, int n_launches, const int* n_tiles, const int* cap,
                             int4* const* tables, hipStream_t s);
hipError_t launch_gemm(Elem e, Epi epi, const GemmArgs& a, const GemmPlan& p, hipStream_t s);
// Dense (single-group) PLAIN GEMM with fp32 output, split along K when the
// tile grid alone would leave the GPU idle; `partial` must hold
// ksplit * T * N floats. splitk_partial_rows_upto(T, ...) * N floats cover
// every batch of at most T rows.
GemmPlan plan_dense_splitk(int64_t T, int N, int K, int chunk);
int64_t splitk_partial_rows_upto(int64_t T, int N, int K, int chunk);
hipError_t launch_splitk_reduce(const GemmArgs& a, int ksplit, hipStream_t s);
// Compute-bound shapes (bf16): 256 x 256 tiles through a 2-stage LDS ring.
GemmPlan plan_gemm_big(Epi epi, int64_t rows_upper, int n_groups, int N);
hipError_t launch_gemm_big(Epi epi, const GemmArgs& a, const GemmPlan& p, hipStream_t s);
// The router GEMM of a large bf16 batch on 256 x 256 tiles split along K
// (gemm_big.hip; ksplit 0 when it does not apply; partial sums of ksplit x T
// rows, at most max(2 T, 131072)), finished by launch_splitk_reduce.
GemmPlan plan_router_big(int64_t T, int N, int K);
// The gate/up GEMM at compute-bound shapes (bf16) on prepacked weights
// (gemm_pf.hip): the same 256 x 256 tiles and schedule as plan_gemm_big
// (big = 2), B read from the packed layout of moe_prepack_weights. SWIGLU only.
GemmPlan plan_gemm_pf(int64_t rows_upper, int n_groups, int inter);
hipError_t launch_gemm_pf(Epi epi, const GemmArgs& a, const GemmPlan& p, hipStream_t s);
// Packs n_experts consecutive gate/up weights [2 inter, K] (bf16) into the
// packed layout.
hipError_t launch_prepack(const void* src, void* dst, int64_t n_experts, int inter, int K, hipStream_t s);
// Packs n_experts consecutive down weights [N, K] (bf16): panels of 64 rows,
// the two 32-row halves in place of the gate and up rows.
hipError_t launch_prepack_down(const void* src, void* dst, int64_t n_experts, int N, int K, hipStream_t s);
// The shared expert (one group of T rows, bf16) on 128 x 128 tiles that fit
// beside the routed decode tiles on a CU (gemm_cores.hip); one persistent
// workgroup per CU (`cus` = compute units of the device).
GemmPlan plan_gemm_cores(Epi epi, int64_t T, int N, int cus);
hipError_t launch_gemm_cores(Epi epi, const GemmArgs& a, const GemmPlan& p, hipStream_t s);

// --- FP8: activation quantisation (K4) and block-scaled grouped GEMM ---------
hipError_t launch_quant_fp8(const void* x_bf16, uint8_t* q, float* scale, int64_t rows, int cols, hipStream_t s);
GemmPlan plan_gemm_fp8(Epi epi, int64_t rows_upper, int n_groups, int64_t expected_rows_per_group, int N);
hipError_t launch_gemm_fp8(Epi epi, const GemmArgs& a, const GemmPlan& p, hipStream_t s);
// Compute-bound shapes (fp8): 256 x 256 tiles staged through LDS.
GemmPlan plan_gemm_fp8_big(Epi epi, int64_t rows_upper, int n_groups, int N);

// --- FP4 (MX) weights: activation quantisation and the scaled-MFMA GEMM -----
hipError_t launch_quant_mx(const void* x_bf16, uint8_t* q, uint8_t* scale, int64_t rows, int cols, hipStream_t s);
GemmPlan plan_gemm_mx(Epi epi, int64_t rows_upper, int n_groups, int64_t expected_rows_per_group, int N);
hipError_t launch_gemm_mx(Epi epi, const GemmArgs& a, const GemmPlan& p, hipStream_t s);

// --- expert load statistics and placement -----------------------------------
hipError_t launch_expert_load(const int32_t* ids, int64_t n, int E, int64_t* load, hipStream_t s);
hipError_t launch_mfma_loop(int64_t iters, unsigned long long* out, double* flops, hipStream_t s);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* out, hipStream_t s);
void plan_placement(const int64_t* load, int E, int ranks, int redundant, int32_t* replicas, int32_t* slot_expert,
                    double* rank_load);

// --- combine (K7) ------------------------------------------------------------
struct CombineArgs {
    const void* rows;         // [R, H]
    const int32_t* inv;       // [T, k]
    const float* w;           // [T, k]
    const float* shared;      // [T, H] fp32 or null
    void* y;                  // [T, H]
    int64_t T;
    int H, k;
    int rows_f32;             // rows are fp32 (else bf16)
    int out_f32;              // y is fp32 (else bf16)
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

}  // namespace moe
