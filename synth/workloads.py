"""The five MoE-layer workloads, as plain parameter dictionaries.

Shapes follow the DeepSeek-V3 layer described in the infra guide "Data
parallelism and expert parallelism" (section 2.1: hidden 7168, 256 routed
experts plus one shared expert, expert intermediate 2048, top-8) and the
Perplexity post "Lower latency and higher throughput with multi-node DeepSeek
deployment" (section "Parallelization techniques > Expert parallelism": each
token goes to 8 of 256 routed experts, one shared expert on every rank, 256/EP
routed experts per GPU).

Keys:
  T            tokens in the batch
  hidden       H
  n_experts    E, global routed experts
  expert_begin, expert_end   the local share [b, e) of routed experts
  top_k        k
  n_group, topk_group        group-limited routing (G groups, keep G_k)
  score_fn     "softmax" or "sigmoid"
  renormalize  gates renormalised over the selected experts
  routed_scale gamma, the routed scaling factor
  inter        I, expert intermediate size
  shared_inter I_s, shared-expert intermediate size (0 = no shared expert)
  dtype        "f32", "bf16", "fp8" or "mxfp4" (weights; activations follow:
               bf16 in, e4m3 at the expert GEMMs for fp8 and mxfp4)
  capacity_factor  <= 0 means no capacity limit
  score_bias   "none", "zero", "normal0.01" or "normal0.1" (selection-only bias)
  router_bias  "none" or "zipf1.1" (linear bias of the router GEMM)
"""

_BASE_DSV3 = dict(
    hidden=7168, n_experts=256, top_k=8, n_group=8, topk_group=4,
    score_fn="sigmoid", renormalize=True, routed_scale=1.0,
    inter=2048, shared_inter=2048, capacity_factor=0.0,
    router_bias="none",
)

WORKLOADS = {
    # Toy fp32 layer: softmax top-2 with renormalised gates, no shared expert.
    "toy_fp32": dict(
        T=2048, hidden=512, n_experts=8, expert_begin=0, expert_end=8, top_k=2,
        n_group=1, topk_group=1, score_fn="softmax", renormalize=True,
        routed_scale=1.0, inter=512, shared_inter=0, dtype="f32",
        capacity_factor=0.0, score_bias="none", router_bias="none"),
    # One GPU's EP8 share (routed experts 0..31) of a DeepSeek-V3 layer, decode.
    "ep8_decode_bf16": dict(_BASE_DSV3, T=2048, expert_begin=0, expert_end=32,
                            dtype="bf16", score_bias="normal0.01"),
    # Whole 256-expert layer on one GPU, decode batch (~16 rows per expert).
    "full_decode_bf16": dict(_BASE_DSV3, T=512, expert_begin=0, expert_end=256,
                             dtype="bf16", score_bias="normal0.01"),
    # Same layer at prefill shape (~512 rows per expert).
    "full_prefill_bf16": dict(_BASE_DSV3, T=16384, expert_begin=0, expert_end=256,
                              dtype="bf16", score_bias="zero"),
    # e4m3 weights with 128x128 block scales, skewed routing, capacity 1.25.
    "fp8_skew": dict(_BASE_DSV3, T=8192, expert_begin=0, expert_end=256,
                     dtype="fp8", score_bias="zero", capacity_factor=1.25,
                     router_bias="zipf1.1"),
    # Whole 256-expert layer, decode batch, with FP4 (MX) expert weights: the
    # weight-bandwidth-bound shape where FP4 halves the bytes again (NVIDIA,
    # "Optimizing DeepSeek R1 throughput on Blackwell", FP4 checkpoint).
    "full_decode_mxfp4": dict(_BASE_DSV3, T=512, expert_begin=0, expert_end=256,
                              dtype="mxfp4", score_bias="normal0.01"),
}

ORDER = ["toy_fp32", "ep8_decode_bf16", "full_decode_bf16", "full_prefill_bf16", "fp8_skew"]


def workload(name, **overrides):
    """A copy of workload `name` with `overrides` applied (e.g. T=64)."""
    w = dict(WORKLOADS[name])
    w.update(overrides)
    w["name"] = name
    return w


def local_experts(w):
    return w["expert_end"] - w["expert_begin"]
