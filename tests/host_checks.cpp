// Host-side checks of libmoe's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitizers.py
// builds and runs it on the CPU; no call here reaches a kernel launch).
//
// Covered: argument validation of every entry point (configs, null and
// misaligned pointers, workspace and packed-buffer sizes, the 4 GiB operand
// limit, the allocation-free entry point's scratch limit), workspace and
// packed-weight sizing over a range of token counts (never shrinking as the
// batch grows), and the placement planner over random loads (replicas,
// slots and loads conserved, imbalance >= 1).
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "moe.h"

static int g_fail = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);   \
            ++g_fail;                                                            \
        }                                                                        \
    } while (0)

static moe_config dsv3(int dtype) {
    moe_config c{};
    c.abi_version = MOE_ABI_VERSION;
    c.hidden = 7168;
    c.n_experts = 256;
    c.expert_begin = 0;
    c.expert_end = 32;
    c.top_k = 8;
    c.n_group = 8;
    c.topk_group = 4;
    c.score_fn = MOE_SCORE_SIGMOID;
    c.renormalize = 1;
    c.routed_scale = 1.0f;
    c.inter = 2048;
    c.shared_inter = 2048;
    c.dtype = dtype;
    c.out_dtype = MOE_DTYPE_BF16;
    c.capacity_factor = 0.0f;
    return c;
}

static void* const FAKE = reinterpret_cast<void*>(uintptr_t{0x10000});   // never dereferenced

static void validation() {
    CHECK(moe_validate_config(nullptr) == MOE_ERR_INVALID_ARG);
    moe_config c = dsv3(MOE_DTYPE_BF16);
    CHECK(moe_validate_config(&c) == MOE_OK);
    c.abi_version = MOE_ABI_VERSION + 1;
    CHECK(moe_validate_config(&c) == MOE_ERR_ABI_MISMATCH);
    // a sweep of configs: every status must be one of the defined codes,
    // and what the header promises must hold
    std::mt19937 rng(7);
    for (int it = 0; it < 20000; ++it) {
        moe_config d{};
        d.abi_version = MOE_ABI_VERSION;
        d.hidden = 128 * static_cast<int>(rng() % 70) - 64 * static_cast<int>(rng() % 2);
        d.n_experts = static_cast<int>(rng() % 600) - 5;
        d.expert_begin = static_cast<int>(rng() % 300) - 5;
        d.expert_end = d.expert_begin + static_cast<int>(rng() % 300) - 5;
        d.top_k = static_cast<int>(rng() % 20) - 1;
        d.n_group = static_cast<int>(rng() % 70) - 1;
        d.topk_group = static_cast<int>(rng() % 70) - 1;
        d.score_fn = static_cast<int>(rng() % 3);
        d.renormalize = static_cast<int>(rng() % 3);
        d.routed_scale = 1.0f;
        d.inter = 128 * static_cast<int>(rng() % 20);
        d.shared_inter = 128 * static_cast<int>(rng() % 20) - 128;
        d.dtype = static_cast<int>(rng() % 5);
        d.out_dtype = static_cast<int>(rng() % 3);
        d.capacity_factor = (rng() % 2) ? 1.25f : 0.0f;
        const int st = moe_validate_config(&d);
        CHECK(st == MOE_OK || st == MOE_ERR_INVALID_ARG || st == MOE_ERR_UNSUPPORTED);
        if (st == MOE_OK) {
            CHECK(d.n_experts % d.n_group == 0);
            CHECK(d.n_group == 1 || d.n_experts / d.n_group >= 2);
            CHECK(1 <= d.topk_group && d.topk_group <= d.n_group);
            CHECK(1 <= d.top_k && d.top_k <= 16 && d.top_k <= d.topk_group * (d.n_experts / d.n_group));
            CHECK(0 <= d.expert_begin && d.expert_begin < d.expert_end && d.expert_end <= d.n_experts);
            CHECK(d.hidden % 128 == 0 && d.inter % 128 == 0 && d.shared_inter % 128 == 0);
            size_t ws = 0;
            CHECK(moe_workspace_bytes(&d, 100, &ws) == MOE_OK && ws > 0);
        }
    }
}

static void sizing() {
    for (int dtype : {MOE_DTYPE_F32, MOE_DTYPE_BF16, MOE_DTYPE_FP8, MOE_DTYPE_MXFP4}) {
        moe_config c = dsv3(dtype);
        c.expert_end = 256;
        size_t prev = 0;
        for (int64_t T = 0; T <= 20000; T += (T < 300 ? 1 : 37)) {
            size_t ws = 0;
            CHECK(moe_workspace_bytes(&c, T, &ws) == MOE_OK);
            CHECK(ws >= prev);
            prev = ws;
        }
        size_t pk = 0;
        const int st = moe_packed_weights_bytes(&c, &pk);
        if (dtype == MOE_DTYPE_BF16) {
            // the routed and shared gate/up weights and the routed down weights, 2 bytes each
            CHECK(st == MOE_OK && pk == size_t{2} * (256 * size_t{2} * 2048 * 7168 + size_t{2} * 2048 * 7168 +
                                                     256 * size_t{7168} * 2048));
        } else {
            CHECK(st == MOE_ERR_UNSUPPORTED);
        }
    }
    moe_config c = dsv3(MOE_DTYPE_BF16);
    size_t ws = 0;
    CHECK(moe_workspace_bytes(&c, -1, &ws) == MOE_ERR_INVALID_ARG);
    CHECK(moe_workspace_bytes(&c, 10, nullptr) == MOE_ERR_INVALID_ARG);
}

static void rejections() {
    moe_config c = dsv3(MOE_DTYPE_BF16);
    moe_weights w{};
    w.w13 = w.w2 = w.shared_w13 = w.shared_w2 = FAKE;
    size_t need = 0;
    CHECK(moe_workspace_bytes(&c, 4, &need) == MOE_OK);
    float* f = static_cast<float*>(FAKE);
    int32_t* i = static_cast<int32_t*>(FAKE);
    // T == 0 is a no-op whatever the pointers
    CHECK(moe_route(&c, 0, nullptr, nullptr, nullptr, nullptr, nullptr) == MOE_OK);
    CHECK(moe_forward(&c, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                      nullptr) == MOE_OK);
    CHECK(moe_forward_noalloc(&c, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr) == MOE_OK);
    // negative or huge T, null pointers, misalignment, small workspaces
    CHECK(moe_route(&c, -1, f, nullptr, i, f, nullptr) == MOE_ERR_INVALID_ARG);
    CHECK(moe_route(&c, int64_t{1} << 40, f, nullptr, i, f, nullptr) == MOE_ERR_INVALID_ARG);
    CHECK(moe_route(&c, 4, nullptr, nullptr, i, f, nullptr) == MOE_ERR_INVALID_ARG);
    CHECK(moe_route(&c, 4, f + 1, nullptr, i, f, nullptr) == MOE_ERR_MISALIGNED);
    CHECK(moe_dispatch(&c, 4, i, nullptr, i, i, i, i, FAKE, need - 1, nullptr) == MOE_ERR_WORKSPACE_TOO_SMALL);
    CHECK(moe_dispatch(&c, 4, i, nullptr, i, i, i, i, nullptr, need, nullptr) == MOE_ERR_INVALID_ARG);
    CHECK(moe_combine(&c, 4, FAKE, nullptr, f, nullptr, FAKE, nullptr) == MOE_ERR_INVALID_ARG);
    CHECK(moe_router_gemm(&c, 4, FAKE, FAKE, nullptr, f, FAKE, 1, nullptr) == MOE_ERR_WORKSPACE_TOO_SMALL);
    moe_weights none{};
    CHECK(moe_expert_ffn(&c, 4, FAKE, i, i, &none, FAKE, FAKE, FAKE, need, nullptr) == MOE_ERR_INVALID_ARG);
    CHECK(moe_expert_ffn(&c, 4, FAKE, i, i, &w, FAKE, nullptr, FAKE, need, nullptr) == MOE_ERR_INVALID_ARG);
    // packed weights: bf16 only, 16-byte aligned
    moe_weights wp = w;
    wp.packed = static_cast<char*>(FAKE) + 8;
    CHECK(moe_forward(&c, 4, FAKE, FAKE, nullptr, nullptr, &wp, FAKE, nullptr, nullptr, FAKE, need, nullptr) ==
          MOE_ERR_INVALID_ARG);
    moe_config c8 = dsv3(MOE_DTYPE_FP8);
    wp.packed = FAKE;
    wp.w13_scale = wp.w2_scale = wp.shared_w13_scale = wp.shared_w2_scale = FAKE;
    CHECK(moe_forward(&c8, 4, FAKE, FAKE, nullptr, nullptr, &wp, FAKE, nullptr, nullptr, FAKE, need, nullptr) ==
          MOE_ERR_INVALID_ARG);
    // prepack: sizes, alignment, dtype
    size_t pk = 0;
    CHECK(moe_packed_weights_bytes(&c, &pk) == MOE_OK);
    CHECK(moe_prepack_weights(&c, &w, FAKE, pk - 1, nullptr) == MOE_ERR_WORKSPACE_TOO_SMALL);
    CHECK(moe_prepack_weights(&c, &w, static_cast<char*>(FAKE) + 16, pk, nullptr) == MOE_ERR_MISALIGNED);
    CHECK(moe_prepack_weights(&c, nullptr, FAKE, pk, nullptr) == MOE_ERR_INVALID_ARG);
    {
        moe_weights no_down = w;               // the down weights are packed too: required
        no_down.w2 = nullptr;
        CHECK(moe_prepack_weights(&c, &no_down, FAKE, pk, nullptr) == MOE_ERR_INVALID_ARG);
    }
    CHECK(moe_prepack_weights(&c8, &w, FAKE, pk, nullptr) == MOE_ERR_UNSUPPORTED);
    // operands past 4 GiB, and the allocation-free entry point's scratch limit
    moe_config full = dsv3(MOE_DTYPE_BF16);
    full.expert_end = 256;
    CHECK(moe_forward(&full, 131073, FAKE, FAKE, nullptr, nullptr, &w, FAKE, nullptr, nullptr, FAKE, 1, nullptr) ==
          MOE_ERR_UNSUPPORTED);
    CHECK(moe_forward(&full, 131072, FAKE, FAKE, nullptr, nullptr, &w, FAKE, nullptr, nullptr, FAKE, 1, nullptr) ==
          MOE_ERR_WORKSPACE_TOO_SMALL);
    CHECK(moe_forward_noalloc(&full, 340, FAKE, FAKE, nullptr, nullptr, &w, FAKE, nullptr, nullptr, nullptr) ==
          MOE_ERR_WORKSPACE_TOO_SMALL);
    // the dispatch error word's diagnostic: argument checks before any HIP call
    int64_t nbad = -1;
    CHECK(moe_dispatch_errors(FAKE, 4096, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
    CHECK(moe_dispatch_errors(static_cast<char*>(FAKE) + 4, 4096, nullptr, &nbad) == MOE_ERR_MISALIGNED);
    CHECK(moe_dispatch_errors(FAKE, 255, nullptr, &nbad) == MOE_ERR_WORKSPACE_TOO_SMALL);
    CHECK(nbad == -1);
    // an invalid config is reported by every entry point
    moe_config bad = dsv3(MOE_DTYPE_BF16);
    bad.n_group = 7;
    CHECK(moe_forward(&bad, 4, FAKE, FAKE, nullptr, nullptr, &w, FAKE, nullptr, nullptr, FAKE, need, nullptr) ==
          MOE_ERR_INVALID_ARG);
    CHECK(moe_expert_load(&bad, 4, i, reinterpret_cast<int64_t*>(FAKE), nullptr) == MOE_ERR_INVALID_ARG);
    CHECK(moe_quantize_fp8(&bad, 4, FAKE, static_cast<uint8_t*>(FAKE), f, nullptr) == MOE_ERR_INVALID_ARG);
    // status strings for every code and an unknown one
    for (int st = -7; st <= 0; ++st) CHECK(moe_status_string(st) != nullptr);
}

static void placement() {
    std::mt19937_64 rng(11);
    for (int it = 0; it < 3000; ++it) {
        const int ranks = 1 + static_cast<int>(rng() % 16);
        const int per = 1 + static_cast<int>(rng() % 12);
        const int redundant = static_cast<int>(rng() % (per * ranks));
        const int E = per * ranks - redundant;
        if (E <= 0) continue;
        std::vector<int64_t> load(E);
        int64_t total = 0;
        for (auto& l : load) {
            l = (rng() % 4 == 0) ? 0 : static_cast<int64_t>(rng() % 100000);
            total += l;
        }
        std::vector<int32_t> replicas(E), slots(E + redundant);
        std::vector<double> rank_load(ranks);
        double imb = 0.0;
        CHECK(moe_eplb_plan(load.data(), E, ranks, redundant, replicas.data(), slots.data(), rank_load.data(),
                            &imb) == MOE_OK);
        int64_t nrep = 0;
        for (int e = 0; e < E; ++e) {
            CHECK(replicas[e] >= 1);
            nrep += replicas[e];
        }
        CHECK(nrep == E + redundant);
        std::vector<int> seen(E, 0);
        for (int32_t s : slots) {
            CHECK(s >= 0 && s < E);
            if (s >= 0 && s < E) ++seen[s];
        }
        for (int e = 0; e < E; ++e) CHECK(seen[e] == replicas[e]);
        double sum = 0.0;
        for (double r : rank_load) sum += r;
        CHECK(sum > total - 1e-6 * (total + 1) && sum < total + 1e-6 * (total + 1));
        CHECK(imb >= 1.0 - 1e-12);
    }
    int64_t l[4] = {1, 2, 3, 4};
    int32_t r[4], s[4];
    double rl[2], imb;
    CHECK(moe_eplb_plan(l, 4, 3, 0, r, s, rl, &imb) == MOE_ERR_INVALID_ARG);   // 4 slots on 3 GPUs
    l[1] = -1;
    CHECK(moe_eplb_plan(l, 4, 2, 0, r, s, rl, &imb) == MOE_ERR_INVALID_ARG);   // negative load
    CHECK(moe_eplb_plan(nullptr, 4, 2, 0, r, s, rl, &imb) == MOE_ERR_INVALID_ARG);
}

int main() {
    validation();
    sizing();
    rejections();
    placement();
    if (g_fail) {
        fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    printf("host checks passed\n");
    return 0;
}
