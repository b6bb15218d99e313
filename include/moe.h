/*
 * moe.h - C ABI of the MI355X (gfx950) MoE layer forward library, libmoe.so.
 *
 * The layer is the DeepSeek-V3/R1-style mixture-of-experts FFN:
 *   route    -> a router GEMM gives per-expert logits; scores, group-limited
 *               top-k and gates pick k experts per token;
 *   dispatch -> tokens are permuted into expert-contiguous order;
 *   experts  -> each local expert runs a SwiGLU FFN on its rows (a grouped
 *               GEMM), plus the shared expert on every token;
 *   combine  -> each token's k expert outputs are un-permuted, weighted by
 *               the gates and summed, and the shared output is added.
 * Sources: Ultralytics glossary "Expert Parallelism" (section "How tokens
 * move between GPUs": route, dispatch, compute, combine; section "Load
 * balancing and capacity": capacity factor, selection-only bias); Perplexity
 * "Lower latency and higher throughput with multi-node DeepSeek deployment"
 * (sections "Expert parallelism", "Roofline > GroupGEMM", "Quantization",
 * "MoE Router"); NVIDIA "Optimizing DeepSeek R1 throughput on Blackwell"
 * (section "MoE layer optimisations": mixed-precision router GEMM, fused
 * group-limited top-k); infra guide "Data parallelism and expert parallelism"
 * (section 2.1: shapes; section 3.1: the four steps).
 *
 * Conventions for every call:
 *  - Pointers marked "device" are device memory owned by the caller; the
 *    library never allocates or frees device memory and keeps no per-call
 *    state. `ws` is a caller-owned device workspace of at least the size
 *    moe_workspace_bytes() reports for the same config and token count.
 *  - Every call is asynchronous and ordered on `stream`; outputs are valid
 *    when the stream reaches that point. No call synchronises or reads
 *    device data on the host, so calls can be captured in a HIP graph.
 *  - Arguments are validated before anything is enqueued: a nonzero return
 *    means nothing was launched. T == 0 is a successful no-op.
 *  - The GEMMs address operand rows with 32-bit byte offsets: a call whose
 *    x [T, H], intermediate rows [T k, I] or [T, I_s], router weight [E, H]
 *    or one expert's [2 I, H] weights would span more than 4 GiB (counted at
 *    4 bytes per element for F32, 2 otherwise) returns MOE_ERR_UNSUPPORTED
 *    (DeepSeek-V3 bf16 shape: from T = 131,073 tokens in one call).
 *  - All arrays are row-major and contiguous; device pointers must be
 *    16-byte aligned.
 *  - Calls that share a workspace must not overlap on different streams.
 *  - Unless both the routed experts and the shared expert take the
 *    256 x 256 tiles (bf16 prefill shapes), moe_expert_ffn and moe_forward
 *    run the shared expert on a second stream of the current device, so that
 *    it overlaps the routed path: forked from `stream` (in moe_forward before
 *    the router GEMM, as it needs only x), its down GEMM ordered after the
 *    routed gate/up GEMM, and joined back into `stream` before its output is
 *    read. That stream and its three events are created on the first such
 *    call on a device and kept until the process ends; enqueueing on them is
 *    serialised by a lock, so calls from several host threads are safe.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 4: the packed weight buffer (moe_prepack_weights) also holds the routed
 * down weights; a buffer packed by an earlier version is too short for it. */
#define MOE_ABI_VERSION 4

/* Status codes returned by every entry point. */
enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,          /* bad config value, NULL pointer, T < 0 */
    MOE_ERR_UNSUPPORTED = -2,          /* valid config outside what the kernels handle */
    MOE_ERR_WORKSPACE_TOO_SMALL = -3,
    MOE_ERR_MISALIGNED = -4,           /* a device pointer not 16-byte aligned */
    MOE_ERR_HIP = -5,                  /* a HIP launch error */
    MOE_ERR_ABI_MISMATCH = -6          /* cfg->abi_version != MOE_ABI_VERSION */
};

/* Router score function. */
enum moe_score_fn {
    MOE_SCORE_SOFTMAX = 0,   /* select on logits; gates = softmax over the selected (or all) */
    MOE_SCORE_SIGMOID = 1    /* s = sigmoid(logit); select on s + score_bias; gates from s */
};

/* Numeric format of weights and activations.
 *  F32  : weights, hidden states, intermediate h and expert output rows fp32.
 *  BF16 : weights, hidden states, h and expert output rows bf16; fp32 accumulate.
 *  FP8  : expert weights e4m3fn with one fp32 scale per 128x128 block
 *         (static); hidden states come in bf16 and are quantised to e4m3 with
 *         one fp32 scale per 1x128 block before the gate/up GEMM, h likewise
 *         before the down GEMM (dynamic); expert output rows bf16; the router
 *         weight stays bf16. (Perplexity, section "Quantization".)
 *  MXFP4: expert weights FP4 (E2M1) with one E8M0 power-of-two scale per 32
 *         consecutive elements along the input dimension (OCP microscaling);
 *         hidden states come in bf16 and are quantised to e4m3 with one E8M0
 *         scale per 1x32 block before the gate/up GEMM, h likewise before the
 *         down GEMM; expert output rows bf16; the router weight stays bf16.
 *         (NVIDIA "Optimizing DeepSeek R1 throughput on Blackwell": the MoE
 *         layers' weights in FP4.) Needs H, I and I_s multiples of 256. */
enum moe_dtype {
    MOE_DTYPE_F32 = 0,
    MOE_DTYPE_BF16 = 1,
    MOE_DTYPE_FP8 = 2,
    MOE_DTYPE_MXFP4 = 3
};

typedef struct moe_config {
    int32_t abi_version;     /* MOE_ABI_VERSION */
    int32_t hidden;          /* H */
    int32_t n_experts;       /* E, routed experts of the whole layer */
    int32_t expert_begin;    /* local share [expert_begin, expert_end) of routed experts */
    int32_t expert_end;
    int32_t top_k;           /* k, experts per token (1..16) */
    int32_t n_group;         /* G, expert groups (E % G == 0); 1 = no group limit */
    int32_t topk_group;      /* G_k, groups kept per token (1..G) */
    int32_t score_fn;        /* enum moe_score_fn */
    int32_t renormalize;     /* 1: gates renormalised over the k selected */
    float routed_scale;      /* gamma, multiplies every gate */
    int32_t inter;           /* I, routed expert intermediate size */
    int32_t shared_inter;    /* I_s, shared expert intermediate size; 0 = none */
    int32_t dtype;           /* enum moe_dtype */
    int32_t out_dtype;       /* MOE_DTYPE_F32 or MOE_DTYPE_BF16: layer output y */
    float capacity_factor;   /* > 0: each local expert keeps at most
                                ceil(cf * T * k / E) pairs, in token order */
} moe_config;

/* Expert weights, canonical nn.Linear (out x in) layout, local experts only.
 *  w13       [E_l, 2I, H]: rows 0..I-1 gate, I..2I-1 up projection
 *  w2        [E_l, H, I]:  down projection
 *  shared_*  the same for the shared expert with I_s ([2 I_s, H], [H, I_s])
 *  *_scale   FP8: fp32 [E_l, 2I/128, H/128], [E_l, H/128, I/128] and
 *            [2 I_s/128, H/128], [H/128, I_s/128];
 *            MXFP4: E8M0 bytes [E_l, 2I, H/32], [E_l, H, I/32] and
 *            [2 I_s, H/32], [H, I_s/32] (8-byte aligned); NULL otherwise.
 * MXFP4 weight rows are packed two E2M1 codes per byte, element 2i in the low
 * nibble: w13 [E_l, 2I, H/2] bytes, w2 [E_l, H, I/2] bytes.
 *  packed    BF16 only, optional (NULL: none): the buffer moe_prepack_weights
 *            filled from these same weights. With it, batches whose routed
 *            GEMMs take the 256 x 256 compute-bound tiles (hundreds of rows
 *            per expert: prefill shapes) stream the routed gate/up and down
 *            weights and the shared gate/up weights from it straight into
 *            registers; every other GEMM still reads the canonical arrays,
 *            which stay required. */
typedef struct moe_weights {
    const void* w13;
    const void* w2;
    const void* w13_scale;
    const void* w2_scale;
    const void* shared_w13;
    const void* shared_w2;
    const void* shared_w13_scale;
    const void* shared_w2_scale;
    const void* packed;
} moe_weights;

int moe_abi_version(void);
const char* moe_status_string(int status);

/* Checks the config alone (host only): E % G == 0, E/G >= 2 when G > 1,
 * 1 <= topk_group <= G, 1 <= k <= min(16, topk_group * E / G),
 * 0 <= begin < end <= E, H % 128 == 0, I % 128 == 0, I_s % 128 == 0,
 * E <= 512, E_l <= 1024. */
int moe_validate_config(const moe_config* cfg);

/* Bytes of workspace that moe_forward (and each stage call) needs for up to
 * max_tokens tokens. Written to *bytes. */
int moe_workspace_bytes(const moe_config* cfg, int64_t max_tokens, size_t* bytes);

/* Prepacked expert weights for the compute-bound grouped GEMM (BF16 layers).
 * The expert FFN is three matrices per expert, gate, up and down (infra guide
 * "Data parallelism and expert parallelism", section 2.1); at prefill shapes
 * its grouped GEMM is bound by the matrix cores (Perplexity, "Roofline >
 * GroupGEMM"), and the 256 x 256 gate/up tiles then stream each weight panel
 * from HBM straight into registers, as MFMA operand fragments in the order
 * they are consumed. The packed buffer holds, 256-byte aligned and in this
 * order: the routed w13 [E_l] blocks, (when shared_inter > 0) the shared
 * w13 block, and the routed w2 [E_l] blocks, each the size of its canonical
 * array. (The shared expert's down projection, whose output is fp32, is read
 * in canonical layout.)
 * A block is a sequence of 64-row panels, each of K/16 steps of 2 KB, each
 * panel's rows in two halves of 32: for a [2I, K] gate/up weight panel p
 * holds gate rows 32p..32p+31 (half 0) and the up rows I + 32p..I + 32p + 31
 * of the same h columns (half 1); for an [H, K] down weight (K = I) panel p
 * holds rows 64p..64p+31 (half 0) and 64p+32..64p+63 (half 1). Element
 * (row n, column k) of half h, with n' its index within the half, sits at
 * byte ((p * K/16 + k/16) * 2 + h) * 1024 + (n' + 32 * ((k/8) % 2)) * 16
 * + (k % 8) * 2 of the block: one lane's 8 consecutive K values per 16 bytes,
 * a wavefront's two 32 x 16 fragments of a K step in 2 KB of consecutive
 * memory.
 *
 * moe_packed_weights_bytes: the packed buffer's size for cfg (BF16 only;
 * other dtypes return MOE_ERR_UNSUPPORTED). Host only.
 * moe_prepack_weights: fills `packed` (device, 256-byte aligned, at least
 * packed_bytes = moe_packed_weights_bytes) from the canonical weights
 * (w13, w2 and, with a shared expert, shared_w13; device). Asynchronous on
 * `stream`; run once, before the weights are used. */
int moe_packed_weights_bytes(const moe_config* cfg, size_t* bytes);
int moe_prepack_weights(const moe_config* cfg, const moe_weights* canonical, void* packed, size_t packed_bytes,
                        hipStream_t stream);

/* Router GEMM: logits[T, E] (fp32) = x[T, H] . w_router[E, H]^T + router_bias.
 * x and w_router are fp32 (F32) or bf16 (BF16, FP8, MXFP4): inputs of the activation
 * type in, fp32 out, no separate cast (NVIDIA, "MoE layer optimisations >
 * mixed I/O RouterGEMM"). router_bias [E] fp32 may be NULL. All device; the
 * workspace holds split-K partial sums. */
int moe_router_gemm(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                    const float* router_bias, float* logits, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* Scores and group-limited top-k (NVIDIA, "Top-K kernel fusion"; Perplexity,
 * "MoE Router"; glossary, "Load balancing and capacity").
 *  logits     [T, E] fp32 device, finite
 *  score_bias [E] fp32 device or NULL: added to the score for selection only
 *  topk_ids   [T, k] int32 device out: global expert ids, slot order =
 *             descending selection score, ties to the lower expert id
 *  topk_w     [T, k] fp32 device out: gates
 * Group score = sum of the two largest selection scores in the group; the G_k
 * best groups are kept (ties to the lower group). Sigmoid gates are
 * s_j / sum_i s_i (unbiased scores, if renormalize) times routed_scale;
 * softmax gates are exp(l_j - max) / sum over the selected (or all) experts.
 * The float32 exp/sigmoid follow a fixed recipe (Cody-Waite reduction,
 * degree-8 Taylor polynomial, ldexp; no fused multiply-add; correctly
 * rounded division), so results are reproducible bit for bit. */
int moe_route(const moe_config* cfg, int64_t T, const float* logits, const float* score_bias,
              int32_t* topk_ids, float* topk_w, hipStream_t stream);

/* Dispatch: a stable permutation of the (token, slot) pairs into
 * expert-contiguous order for the local experts (Perplexity, "MoE Router":
 * dense dispatch needs the routing aggregated per expert; glossary: capacity).
 * Pairs p = t*k + j are taken in increasing p. All int32 device:
 *  topk_ids   [T, k] in
 *  raw_counts [E_l] out (may be NULL): local pairs per expert before capacity
 *  counts     [E_l] out: kept rows per expert (min(raw, C))
 *  offsets    [E_l + 1] out: exclusive prefix of counts; offsets[E_l] = R
 *  perm       [T*k] out: perm[row] = p for rows 0..R-1 (rest untouched)
 *  inv        [T*k] out: inv[p] = row, or -1 for non-local or dropped pairs
 * An expert id outside [0, E) is treated as non-local, and counted in the
 * workspace's error word (see moe_dispatch_errors). */
int moe_dispatch(const moe_config* cfg, int64_t T, const int32_t* topk_ids, int32_t* raw_counts,
                 int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                 void* ws, size_t ws_bytes, hipStream_t stream);

/* Expert FFNs as grouped GEMMs (Perplexity, "Roofline > GroupGEMM";
 * infra guide section 2.1): for every row r of local expert e,
 *   h = silu(x_t W_gate[e]^T) * (x_t W_up[e]^T),  out_rows[r] = h W_down[e]^T
 * with t = perm[r] / k; and for every token, the shared expert's output in
 * shared_out[t] (if shared_inter > 0). Group sizes are read from `offsets`
 * on the device, so no host synchronisation is needed.
 *  x          [T, H] device, activation type (bf16 for FP8 and MXFP4)
 *  perm, offsets  from moe_dispatch
 *  out_rows   [T*k, H] device out (fp32 for F32, bf16 otherwise: the rows are
 *             what the combine exchange carries); rows >= R untouched
 *  shared_out [T, H] fp32 device out; required iff shared_inter > 0 */
int moe_expert_ffn(const moe_config* cfg, int64_t T, const void* x, const int32_t* perm,
                   const int32_t* offsets, const moe_weights* weights, void* out_rows,
                   void* shared_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Combine (glossary step 4; infra guide section 3.1 step 4):
 *   y[t] = shared_out[t] + sum_j [inv[t,j] >= 0] * topk_w[t,j] * out_rows[inv[t,j]]
 * summed in fp32; dropped and non-local pairs add nothing (no renormalisation).
 * out_rows [T*k, H] as moe_expert_ffn writes it: all T*k rows must be
 * allocated, since the kernel may read row 0 (and discard it) for a pair
 * with no row. y [T, H] device out in cfg->out_dtype; shared_out [T, H] fp32
 * or NULL. */
int moe_combine(const moe_config* cfg, int64_t T, const void* out_rows, const int32_t* inv,
                const float* topk_w, const void* shared_out, void* y, hipStream_t stream);

/* FP8 activation quantisation (Perplexity, section "Quantization": dynamic
 * scales per 1x128 vector, computed online): for each row and each block of
 * 128 columns, a = max |x|; scale = a / 448 and codes = e4m3(x * (448 / a))
 * (OCP E4M3FN, round to nearest even; every step one float32 operation),
 * or scale 1 and zero codes when a == 0.
 *  x [rows, H] bf16 device; q [rows, H] uint8 codes out; scale [rows, H/128]
 *  fp32 out. moe_expert_ffn and moe_forward apply the same quantisation to x
 *  internally when cfg->dtype is MOE_DTYPE_FP8. */
int moe_quantize_fp8(const moe_config* cfg, int64_t rows, const void* x, uint8_t* q, float* scale,
                     hipStream_t stream);

/* MX activation quantisation for MXFP4 layers (OCP microscaling, the
 * activation side of FP4 expert weights): for each row and each block of 32
 * columns, X = floor(log2(max |x|)) - 8 clamped to [-127, 127] (-127 for an
 * all-zero block); codes = e4m3(x * 2**-X) (OCP E4M3FN, round to nearest
 * even, saturating at +-448; the product is exact); scale code = X + 127.
 *  x [rows, H] bf16 device; q [rows, H] uint8 codes out; scale [rows, H/32]
 *  uint8 E8M0 out. cfg->dtype must be MOE_DTYPE_MXFP4; moe_expert_ffn and
 *  moe_forward apply the same quantisation to x internally. */
int moe_quantize_mx(const moe_config* cfg, int64_t rows, const void* x, uint8_t* q, uint8_t* scale,
                    hipStream_t stream);

/* The whole layer: router GEMM, route, dispatch, experts, combine, in the
 * order of the four steps (Ultralytics glossary "Expert Parallelism", section
 * "How tokens move between GPUs": route, dispatch, compute, combine; infra
 * guide "Data parallelism and expert parallelism", section 3.1), with the
 * shared expert added to every token (Perplexity, "Expert parallelism"). One
 * GPU holds the experts [expert_begin, expert_end): dispatch and combine are
 * local permutations, and y is that share's partial output plus the shared
 * expert's.
 *  x [T, H], w_router [E, H] (activation type; bf16 for FP8 and MXFP4), router_bias [E]
 *  and score_bias [E] fp32 or NULL, weights as above; y [T, H] out.
 *  logits_out [T, E] fp32 and topk_ids_out [T, k] int32, if not NULL, receive
 *  the router logits and expert ids. */
int moe_forward(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                const float* router_bias, const float* score_bias, const moe_weights* weights,
                void* y, float* logits_out, int32_t* topk_ids_out,
                void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_forward_noalloc: moe_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid it). Same arguments and result as moe_forward, less the workspace:
 * the layer's scratch lives in a device array of the library's own, of
 * MOE_NOALLOC_SCRATCH_BYTES, one per GPU, held until the process ends. A
 * batch whose workspace (moe_workspace_bytes) exceeds that returns
 * MOE_ERR_WORKSPACE_TOO_SMALL before anything is launched (DeepSeek-V3 bf16
 * shape: up to 339 tokens per call). The call allocates nothing and
 * creates no stream or event: the shared expert runs on `stream` after the
 * routed experts, with the kernels moe_forward uses, so y equals
 * moe_forward's bit for bit. The array's device address is looked up once
 * per device, on the first call with that device current. All calls on one
 * GPU share its array: calls that overlap on one GPU (two streams, or two
 * host threads) race, and must be ordered by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_forward_noalloc(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                        const float* router_bias, const float* score_bias, const moe_weights* weights,
                        void* y, float* logits_out, int32_t* topk_ids_out, hipStream_t stream);

/* moe_dispatch_errors: a diagnostic, never on the layer's path. Every
 * dispatch (moe_dispatch, and the dispatch step of moe_forward and
 * moe_forward_noalloc) counts the topk_ids entries outside [0, E) it meets
 * and writes that count into an error word at the start of its workspace;
 * such pairs are dropped (they reach no expert). This call waits for
 * `stream` (hipStreamSynchronize), then copies the word of the last
 * dispatch enqueued on that workspace before it into *bad_ids.
 *  ws        the workspace the dispatch ran on (device), or NULL for the
 *            array of moe_forward_noalloc on the current device
 *  ws_bytes  its size (at least 256; ignored when ws is NULL)
 * Before the first dispatch on a caller's workspace the word is undefined;
 * a call with T == 0 launches nothing and leaves it unchanged. Errors:
 * INVALID_ARG (bad_ids NULL), MISALIGNED, WORKSPACE_TOO_SMALL, HIP. */
int moe_dispatch_errors(const void* ws, size_t ws_bytes, hipStream_t stream, int64_t* bad_ids);

/* ---- Expert load statistics and placement ----------------------------------
 * Infra guide "Data parallelism and expert parallelism", section 5: under
 * expert parallelism every layer waits for the GPU that received the most
 * tokens; the load each expert receives is recorded every step (5.3) and the
 * experts are periodically re-placed, the hottest replicated (5.2, 5.3).
 *
 * moe_expert_load: adds to load[e] (device int64 [n_experts], 8-byte
 * aligned; the caller zeroes it to start a window) the number of (token,
 * slot) pairs among topk_ids (device int32 [T, top_k], as moe_route writes
 * them) that chose expert e, for every global expert e (the router sees all
 * experts whatever share this GPU holds). Exact integer counts.
 *
 * moe_eplb_plan (host only; all pointers are host memory): from per-expert
 * loads [n_experts] (>= 0), places n_experts + n_redundant expert replicas on
 * n_ranks GPUs, (n_experts + n_redundant) / n_ranks each (must divide
 * evenly). Extra replicas go one at a time to the expert with the largest
 * load per replica; then the replicas, heaviest first (load / replicas),
 * go to the least-loaded GPU with a free slot. Ties: lowest expert id,
 * lowest GPU index; equal replica loads keep (expert, replica) order.
 * Writes replicas[n_experts], slot_expert[n_experts + n_redundant] (GPU g's
 * slots are [g S, (g + 1) S), S = slots per GPU, in placement order),
 * rank_load[n_ranks] (sum of load / replicas over the GPU's slots) and
 * *imbalance = max rank load / mean rank load (1 = balanced; section 5.1).
 * Returns MOE_ERR_INVALID_ARG on null pointers, non-positive counts, a
 * negative load or slots that do not divide evenly. */
int moe_expert_load(const moe_config* cfg, int64_t T, const int32_t* topk_ids, int64_t* load, hipStream_t stream);
int moe_eplb_plan(const int64_t* load, int n_experts, int n_ranks, int n_redundant, int32_t* replicas,
                  int32_t* slot_expert, double* rank_load, double* imbalance);

/* ---- Diagnostics: per-stage timing with HIP events ------------------------
 * Not part of the layer. moe_profile_enable(n) creates 2n HIP events and
 * starts recording: from then on every stage of every call records a start
 * and a stop event on its stream (at most n stages are recorded; later ones
 * are not). moe_profile_enable(0) stops and destroys the events;
 * moe_profile_reset() forgets what was recorded. moe_profile_select(mask)
 * limits recording to the stages whose bit is set (bit s: stage s; all by
 * default, kept across enable calls), so that a timed run can time one
 * kernel without events around the others. moe_profile_query(stage) waits
 * for the recorded events of that stage and returns their summed elapsed
 * time and how many were recorded. Single-threaded use only. */
enum moe_stage {
    MOE_STAGE_ROUTER_GEMM = 0,
    MOE_STAGE_ROUTE = 1,
    MOE_STAGE_DISPATCH = 2,
    MOE_STAGE_GATE_UP = 3,          /* routed experts: gate/up GEMM + SwiGLU */
    MOE_STAGE_DOWN = 4,             /* routed experts: down GEMM */
    MOE_STAGE_SHARED_GATE_UP = 5,
    MOE_STAGE_SHARED_DOWN = 6,
    MOE_STAGE_COMBINE = 7,
    MOE_STAGE_QUANT = 8,            /* FP8, MXFP4: activation quantisation of x */
    MOE_STAGE_COUNT = 9
};
int moe_profile_enable(int max_records);
int moe_profile_reset(void);
int moe_profile_select(unsigned stage_mask);
int moe_profile_query(int stage, double* total_ms, int* count);

/* ---- Diagnostics: the matrix-core rate the chip sustains -------------------
 * Not part of the layer; a yardstick for the grouped GEMMs' MFMA fraction.
 * moe_mfma_loop launches two workgroups of four wavefronts per compute unit;
 * each wavefront runs `iters` (1 .. 2^40) iterations of four independent
 * v_mfma_f32_32x32x16_bf16 chains on pseudo-random bf16 operands, and no
 * memory traffic. *flops (host) receives the FLOPs the launch performs.
 * out (device uint64 [3], 8-byte aligned) receives, for wavefront 0 of
 * workgroup 0: the shader-clock ticks and the 100 MHz real-time ticks its
 * loop took (their ratio times 100 MHz is the shader clock it ran at), and a
 * checksum of its accumulators. The caller times the launch (stream-ordered
 * and asynchronous like every call here). */
int moe_mfma_loop(int64_t iters, uint64_t* out, double* flops, hipStream_t stream);

/* moe_stream_read: reads the `bytes` (a multiple of 16, >= 0) of device
 * buffer src (16-byte aligned) once, one workgroup per compute unit, each
 * taking 64 KB blocks of consecutive memory (sixteen 16-byte loads in flight
 * per lane), and writes almost nothing (out, device uint32 [1], is
 * written only if the XOR of the data equals 0x9e3779b9); timing it gives
 * the rate at which this device streams weights in from HBM. bytes == 0 is
 * a no-op. Not part of the layer. */
int moe_stream_read(const void* src, int64_t bytes, uint32_t* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
