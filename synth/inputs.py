"""Seeded synthetic tensors for the MoE workloads.

Recipe (the pages name no dataset for this layer; these stand in for it):
  * hidden states x ~ N(0, 1);
  * router weight W_r [E, H] and expert weights ~ N(0, 1/fan_in), fan_in = H
    for W_r and the gate/up stack W13 [E_l, 2I, H], I for the down projection
    W2 [E_l, H, I]; the shared expert uses the same rule;
  * selection-only score bias b_e: absent, zero, or N(0, s^2) with s = 0.01
    (decode workloads: it changes the selection of about half the tokens while
    the load stays near-uniform, as a balancing bias intends) or s = 0.1;
  * router linear bias c_e: absent, or a Zipf(s = 1.1) popularity offset
    -1.1 * ln(rank_e) with rank_e = 1 + a seeded permutation of the experts;
  * bf16 tensors are the float32 draws rounded to nearest-even by torch;
  * fp8 weights are e4m3fn codes with one float32 scale per 128x128 block,
    scale = block amax / 448, produced by torch's own float8 cast;
  * mxfp4 weights are drawn directly as codes, not quantised from floats:
    E2M1 codes two to a byte (element 2i in the low nibble), the sign fair,
    the magnitude from a fixed table shaped like a normal sample that fills
    the E2M1 range, and one E8M0 scale per 32 elements along the input
    dimension, 2**floor(l) or 2**(floor(l) + 1) at random with
    l = log2(std / rms(table)), so that the weights' RMS is about the same
    1/sqrt(fan_in).

Every tensor has its own torch.Generator, seeded from
numpy.random.SeedSequence(seed, spawn_key=(tensor_id, global_expert)), so any
expert can be regenerated alone and an expert-parallel share holds exactly the
same experts as the whole layer. Draws on a CUDA device use torch's device
generator (fast at full size); draws on the CPU use the CPU generator. The two
give different numbers, so both sides of a comparison always take their
inputs from one call.
"""
import math

import numpy as np
import torch

from .workloads import local_experts

_TENSOR_IDS = {"x": 1, "w_router": 2, "score_bias": 3, "router_bias": 4,
               "w13": 5, "w2": 6, "shared_w13": 7, "shared_w2": 8}

FP8_MAX = 448.0
BLOCK = 128


def _gen(device, seed, tensor, expert=0):
    ss = np.random.SeedSequence(seed, spawn_key=(_TENSOR_IDS[tensor], expert))
    s = int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _normal(shape, std, device, seed, tensor, expert=0):
    g = _gen(device, seed, tensor, expert)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def _block_fp8(w):
    """float32 [N, K] -> (e4m3fn codes [N, K], float32 scales [N/128, K/128])."""
    n, k = w.shape
    blocks = w.reshape(n // BLOCK, BLOCK, k // BLOCK, BLOCK)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (blocks / scale[:, None, :, None]).clamp_(-FP8_MAX, FP8_MAX)
    return q.reshape(n, k).to(torch.float8_e4m3fn), scale.contiguous()


def zipf_router_bias(n_experts, s=1.1, seed=0):
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(_TENSOR_IDS["router_bias"], 0)))
    rank = 1 + rng.permutation(n_experts)
    return torch.tensor(-s * np.log(rank.astype(np.float64)), dtype=torch.float32)


# Magnitude distribution of the synthetic E2M1 codes 0..7 (values 0, 0.5, 1,
# 1.5, 2, 3, 4, 6): about what a normal sample scaled so that its largest
# value reaches 4..8 looks like on that grid.
FP4_MAG_PROBS = (0.07, 0.14, 0.14, 0.13, 0.18, 0.15, 0.13, 0.06)
FP4_MAG_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
MX_BLOCK = 32


def _fp4_codes(shape, std, device, seed, tensor, expert):
    """Random packed E2M1 codes [N, K/2] and E8M0 scales [N, K/32] (uint8)."""
    n, k = shape
    g = _gen(device, seed, tensor, expert)
    cdf = torch.tensor(np.cumsum(FP4_MAG_PROBS)[:-1], dtype=torch.float32, device=device)
    mag = torch.bucketize(torch.rand((n, k), generator=g, device=device), cdf, right=True)
    sign = (torch.rand((n, k), generator=g, device=device) < 0.5).to(torch.int64) << 3
    codes = (mag | sign).to(torch.uint8)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    rms = math.sqrt(sum(p * v * v for p, v in zip(FP4_MAG_PROBS, FP4_MAG_VALUES)))
    lg = math.log2(std / rms)
    base = math.floor(lg)
    up = (torch.rand((n, k // MX_BLOCK), generator=g, device=device) < (lg - base)).to(torch.int64)
    scales = (127 + base + up).to(torch.uint8)
    return packed.contiguous(), scales.contiguous()


def _weight_dtype(w):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.bfloat16,
            "mxfp4": torch.bfloat16}[w["dtype"]]


def make_inputs(w, device="cpu", seed=0):
    """All input tensors of workload dict `w` on `device`.

    Returns a dict with x, w_router, router_bias (or None), score_bias (or None),
    w13, w2, shared_w13, shared_w2 (None when there is no shared expert) and,
    for fp8 and mxfp4, w13_scale, w2_scale, shared_w13_scale, shared_w2_scale.
    mxfp4 weights are uint8: packed codes [.., N, K/2], scales [.., N, K/32].
    """
    T, H, E, I = w["T"], w["hidden"], w["n_experts"], w["inter"]
    Is = w["shared_inter"]
    El = local_experts(w)
    b0 = w["expert_begin"]
    act_dtype = _weight_dtype(w)
    fp8 = w["dtype"] == "fp8"
    fp4 = w["dtype"] == "mxfp4"
    out = {}

    out["x"] = _normal((T, H), 1.0, device, seed, "x").to(act_dtype)
    out["w_router"] = _normal((E, H), 1.0 / math.sqrt(H), device, seed, "w_router").to(act_dtype)

    sb = w.get("score_bias", "none")
    if sb == "none":
        out["score_bias"] = None
    elif sb == "zero":
        out["score_bias"] = torch.zeros(E, dtype=torch.float32, device=device)
    elif sb in ("normal0.01", "normal0.1"):
        out["score_bias"] = _normal((E,), float(sb[6:]), device, seed, "score_bias")
    else:
        raise ValueError(sb)

    rb = w.get("router_bias", "none")
    if rb == "none":
        out["router_bias"] = None
    elif rb == "zipf1.1":
        out["router_bias"] = zipf_router_bias(E, 1.1, seed).to(device)
    else:
        raise ValueError(rb)

    def expert_stack(name, n_rows, n_cols, experts, std):
        if fp4:
            codes = torch.empty((len(experts), n_rows, n_cols // 2), dtype=torch.uint8, device=device)
            scales = torch.empty((len(experts), n_rows, n_cols // MX_BLOCK), dtype=torch.uint8, device=device)
            for i, e in enumerate(experts):
                codes[i], scales[i] = _fp4_codes((n_rows, n_cols), std, device, seed, name, e)
            return codes, scales
        if fp8:
            codes = torch.empty((len(experts), n_rows, n_cols), dtype=torch.float8_e4m3fn, device=device)
            scales = torch.empty((len(experts), n_rows // BLOCK, n_cols // BLOCK), dtype=torch.float32, device=device)
        else:
            codes = torch.empty((len(experts), n_rows, n_cols), dtype=act_dtype, device=device)
            scales = None
        for i, e in enumerate(experts):
            t = _normal((n_rows, n_cols), std, device, seed, name, e)
            if fp8:
                q, s = _block_fp8(t)
                codes[i].copy_(q)
                scales[i].copy_(s)
            else:
                codes[i].copy_(t)
            del t
        return codes, scales

    experts = list(range(b0, b0 + El))
    out["w13"], out["w13_scale"] = expert_stack("w13", 2 * I, H, experts, 1.0 / math.sqrt(H))
    out["w2"], out["w2_scale"] = expert_stack("w2", H, I, experts, 1.0 / math.sqrt(I))
    if Is > 0:
        s13, s13s = expert_stack("shared_w13", 2 * Is, H, [0], 1.0 / math.sqrt(H))
        s2, s2s = expert_stack("shared_w2", H, Is, [0], 1.0 / math.sqrt(Is))
        out["shared_w13"], out["shared_w2"] = s13[0], s2[0]
        out["shared_w13_scale"] = s13s[0] if (fp8 or fp4) else None
        out["shared_w2_scale"] = s2s[0] if (fp8 or fp4) else None
    else:
        out["shared_w13"] = out["shared_w2"] = None
        out["shared_w13_scale"] = out["shared_w2_scale"] = None
    return out
