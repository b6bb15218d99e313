"""Plain CPU oracle of the DeepSeek-V3/R1-style MoE layer forward.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import this module. The HIP path never calls it and shares
no code with it.

What it computes, stage by stage, with the passage each stage follows:

  route     Ultralytics glossary "Expert Parallelism", section "How tokens move
            between GPUs" (step 1: score every expert, keep the top k) and
            section "Load balancing and capacity" (a per-expert bias that only
            changes which experts are selected); NVIDIA "Optimizing DeepSeek R1
            throughput on Blackwell", section "MoE layer optimisations > Top-K
            kernel fusion" (pick expert groups first, then the top 8 inside
            them, with a bias and a scaling factor); Perplexity "Lower latency
            and higher throughput with multi-node DeepSeek deployment", section
            "MoE Router" (Mixtral routing is the special case where every group
            is kept; sparse kernels take per-token top-k ids and scores).
  dispatch  same Perplexity section (dense dispatch/combine needs the routing
            aggregated per expert) and the glossary's capacity factor (each
            expert takes at most a fixed multiple of its equal share; overflow
            tokens skip that expert).
  experts   infra guide "Data parallelism and expert parallelism", section 2.1
            (an expert is three matrices gate, up, down) and Perplexity section
            "Quantization" (SiLU activation; FP8 weights with static scales per
            128x128 block, activations with dynamic scales per 1x128 vector).
            FP4 expert weights: NVIDIA "Optimizing DeepSeek R1 throughput on
            Blackwell", section on the FP4 checkpoint (the MoE layers' weights
            are FP4). The pages fix no FP4 encoding; the reading here is the
            OCP microscaling (MX) one: E2M1 elements, one E8M0 power-of-two
            scale per 32 consecutive elements along the reduction dimension;
            activations e4m3 with the same 32-element power-of-two scales.
  combine   glossary step 4 and infra guide section 3.1 step 4 (outputs come
            back and are summed weighted by the router scores); the shared
            expert sees every token and its output is added (Perplexity,
            "Expert parallelism").

Precision. Expert and combine arithmetic is fp64 on the exact input values.
Routing decisions (an argmax over floating-point scores) are taken in float32
with the recipe below, step for step, so that the GPU can match them bit for
bit. Between stages the oracle rounds to the carrier type the layer uses: the
intermediate activation h to the activation type (bf16 round-to-nearest-even,
e4m3 with 1x128 scales, or MX e4m3 with 32-element scales), and each routed
expert's output row to bf16 when activations are bf16, fp8 or mxfp4 (the
combine exchange carries BF16, infra guide
section 3.2). The shared expert's output never leaves the token's GPU and is
kept unrounded.

Readings where the pages are silent:
  * group score = sum of the two largest selection scores in the group;
  * ties (experts and groups) go to the lower index; slots hold experts in
    selection order (descending score);
  * sigmoid gates use the unbiased score, renormalised over the k selected,
    then times routed_scale;
  * softmax routing selects on the logits (a strictly monotone map of the
    probabilities); gates are exp(l_j - l_0) / sum_i exp(l_i - l_0) over the
    selected, or over all experts when renormalize is off;
  * dispatch order is stable by (expert, token, slot); capacity is
    C = ceil(cf * T * k / E) with the global E, taken in token order; dropped
    pairs contribute nothing and the gates are not renormalised.

exp and sigmoid follow a fixed float32 recipe (Cody and Waite 1980 range
reduction, Taylor polynomial in Horner form, ldexp), every step one IEEE
float32 operation; see exp_f32 and sigmoid_f32.

Parity pins live in tests/test_oracle_*.py; every function here is pinned.
"""
import math
from dataclasses import dataclass, field

import numpy as np

F32 = np.float32

# ---------------------------------------------------------------------------
# Configuration (a plain record; built from a workload dictionary)
# ---------------------------------------------------------------------------


@dataclass
class Config:
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    n_group: int = 1
    topk_group: int = 1
    score_fn: str = "softmax"
    renormalize: bool = True
    routed_scale: float = 1.0
    shared_inter: int = 0
    expert_begin: int = 0
    expert_end: int = -1
    capacity_factor: float = 0.0
    act: str = "f32"          # "f32", "bf16", "fp8" or "mxfp4"

    def __post_init__(self):
        if self.expert_end < 0:
            self.expert_end = self.n_experts

    @property
    def n_local(self):
        return self.expert_end - self.expert_begin

    @classmethod
    def from_workload(cls, w):
        return cls(hidden=w["hidden"], n_experts=w["n_experts"], top_k=w["top_k"],
                   inter=w["inter"], n_group=w["n_group"], topk_group=w["topk_group"],
                   score_fn=w["score_fn"], renormalize=bool(w["renormalize"]),
                   routed_scale=float(w["routed_scale"]), shared_inter=w["shared_inter"],
                   expert_begin=w["expert_begin"], expert_end=w["expert_end"],
                   capacity_factor=float(w["capacity_factor"]), act=w["dtype"])


# ---------------------------------------------------------------------------
# float32 exp / sigmoid recipe (decides the routing, so fixed step by step)
# ---------------------------------------------------------------------------

# Cody-Waite split of ln 2: the high part has 15 significant bits, so n * LN2_HI
# is exact for |n| < 512.
LN2_HI = F32(0.693145751953125)
LN2_LO = F32(math.log(2.0) - 0.693145751953125)
LOG2E = F32(1.0 / math.log(2.0))
EXP_ARG_MIN = F32(-87.0)
# Taylor coefficients 1/j! for j = 8 .. 0, each rounded to float32.
EXP_COEFFS = [F32(1.0 / math.factorial(j)) for j in range(8, -1, -1)]


def exp_f32(y):
    """e**y for float32 y <= 0, by the fixed recipe.

    y is clamped to >= -87 (so every result is a normal float32); then
    n = rint(y * log2 e); r = (y - n*LN2_HI) - n*LN2_LO; p = degree-8 Taylor
    polynomial of e**r in Horner form; result = ldexp(p, n). Every step is
    one float32 operation (no fused multiply-add).
    """
    y = np.maximum(np.asarray(y, dtype=F32), EXP_ARG_MIN)
    n = np.rint(y * LOG2E).astype(F32)
    r = (y - n * LN2_HI) - n * LN2_LO
    p = np.full_like(r, EXP_COEFFS[0])
    for c in EXP_COEFFS[1:]:
        p = p * r + c
    return np.ldexp(p, n.astype(np.int32)).astype(F32)


def sigmoid_f32(x):
    """Logistic function in float32 by the fixed recipe.

    x >= 0: 1 / (1 + exp_f32(-x));  x < 0: e / (1 + e) with e = exp_f32(x).
    Division is the correctly rounded IEEE float32 division.
    """
    x = np.asarray(x, dtype=F32)
    pos = x >= 0
    e = exp_f32(np.where(pos, -x, x))
    one = F32(1.0)
    den = one + e
    return np.where(pos, one / den, e / den).astype(F32)


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def bf16_round(v):
    """Round to the nearest bfloat16 value (ties to even); returns float64."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                 # v = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # 8 significant bits


def e4m3_decode(codes):
    """OCP E4M3FN code (uint8) -> value (float64): bias 7, 3 mantissa bits,
    exponent field 0 is subnormal (m/8 * 2**-6), S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    val = np.where(ex == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * np.exp2(ex - 7.0))
    val = np.where((ex == 0xF) & (man == 0x7), np.nan, val)
    return sign * val


def e4m3_round(v):
    """Round to the nearest E4M3FN value, ties to even, saturating at +-448.

    With a = m * 2**e (0.5 <= m < 1) the spacing of E4M3 values around a is
    2**(max(e - 1, -6) - 3): three mantissa bits, and a fixed spacing of 2**-9
    in the subnormal range below 2**-6.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)
    q = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    r = np.minimum(np.rint(a / q) * q, 448.0)
    return np.where(v < 0, -r, r)


def quantize_fp8_rows(v):
    """Per (row, 128-column block) dynamic quantisation, in float32.

    a = max |v| over the block; a == 0 -> codes 0, scale 1; otherwise
    inv = 448 / a, q = e4m3_round(v * inv), scale = a / 448 (each a float32
    operation). A block so small that 448 / a overflows float32 (a below
    about 2**-119) takes the largest finite float32 as inv instead, so its
    codes stay finite. Returns (q as float64 values, scales float32
    [rows, cols/128]).
    """
    v = np.asarray(v, dtype=F32)
    rows, cols = v.shape
    blk = v.reshape(rows, cols // 128, 128)
    a = np.max(np.abs(blk), axis=2)
    nz = a > 0
    safe = np.where(nz, a, F32(1.0))
    with np.errstate(over="ignore"):
        inv = (F32(448.0) / safe).astype(F32)
    inv = np.minimum(inv, F32(np.finfo(F32).max))   # a < 2**-119: 448 / a overflows
    prod = (blk * inv[:, :, None]).astype(F32)
    q = np.where(nz[:, :, None], e4m3_round(prod), 0.0)
    scale = np.where(nz, (safe / F32(448.0)).astype(F32), F32(1.0)).astype(F32)
    return q.reshape(rows, cols), scale


def dequant_block_weight(codes, scales):
    """e4m3 codes [N, K] with float32 scales [N/128, K/128] -> float64 [N, K]."""
    w = e4m3_decode(codes)
    n, k = w.shape
    s = np.asarray(scales, dtype=np.float64)
    return (w.reshape(n // 128, 128, k // 128, 128) * s[:, None, :, None]).reshape(n, k)


# ---------------------------------------------------------------------------
# Microscaling (MX) formats: FP4 expert weights, e4m3 activations
# ---------------------------------------------------------------------------

MX_BLOCK = 32
E4M3_EMAX = 8          # largest e4m3 value 448 = 1.75 * 2**8
E2M1_EMAX = 2          # largest e2m1 value 6 = 1.5 * 2**2


def e2m1_decode(codes):
    """E2M1 code (0..15) -> value (float64): sign bit 3, two exponent bits
    with bias 1, one mantissa bit; exponent field 0 is subnormal (m * 0.5)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    ex = (c >> 1) & 0x3
    man = c & 0x1
    val = np.where(ex == 0, man * 0.5, (1.0 + man / 2.0) * np.exp2(ex - 1.0))
    return sign * val


def e8m0_decode(codes):
    """E8M0 scale code -> 2**(code - 127) (float64); code 255 is NaN."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def unpack_fp4(packed):
    """[..., K/2] bytes -> [..., K] E2M1 codes; element 2i is the low nibble of
    byte i and element 2i+1 the high nibble."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def dequant_mx_weight(packed, scales):
    """FP4 weight [N, K/2] bytes with E8M0 scales [N, K/32] -> float64 [N, K]:
    element (n, k) is e2m1(code) * 2**(scale[n, k // 32] - 127)."""
    v = e2m1_decode(unpack_fp4(packed))
    n, k = v.shape
    s = e8m0_decode(scales)
    return (v.reshape(n, k // MX_BLOCK, MX_BLOCK) * s[:, :, None]).reshape(n, k)


def mx_scale_exponent(amax, emax=E4M3_EMAX):
    """Shared exponent of an MX block: floor(log2(amax)) - emax, kept within
    the E8M0 range [-127, 127]; an all-zero block takes -127 (its codes are
    zero whatever the scale)."""
    a = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(a)                 # a = m * 2**e with 0.5 <= m < 1: floor(log2 a) = e - 1
    x = np.where(a > 0, e - 1 - emax, -127)
    return np.clip(x, -127, 127).astype(np.int64)


def quantize_mx_rows(v):
    """Per (row, 32-column block) MX e4m3 quantisation of float32 values.

    X = mx_scale_exponent(max |v| over the block); each element becomes
    e4m3_round(v * 2**-X) (the product is exact: a power of two), saturating
    at +-448. Returns (q as float64 e4m3 values, scale codes uint8 X + 127,
    [rows, cols/32]).
    """
    v = np.asarray(v, dtype=F32).astype(np.float64)
    rows, cols = v.shape
    blk = v.reshape(rows, cols // MX_BLOCK, MX_BLOCK)
    x = mx_scale_exponent(np.max(np.abs(blk), axis=2))
    q = e4m3_round(np.ldexp(blk, -x[:, :, None]))
    return q.reshape(rows, cols), (x + 127).astype(np.uint8)


def dequant_mx_rows(q, scale_codes):
    """Values of MX-quantised rows: q [rows, cols] times 2**(code - 127) per
    32-column block."""
    rows, cols = q.shape
    s = e8m0_decode(scale_codes)
    return (np.asarray(q, dtype=np.float64).reshape(rows, cols // MX_BLOCK, MX_BLOCK) * s[:, :, None]).reshape(rows, cols)


# ---------------------------------------------------------------------------
# Stage 1: router GEMM
# ---------------------------------------------------------------------------

def router_logits(x, w_router, router_bias=None, work=np.float64):
    """logits = x W_r^T (+ c), in fp64 (returned as float64). `work` is the
    matmul's arithmetic type: fp64 for every parity use; the CPU baseline
    timing alone passes float32."""
    l = (np.asarray(x, dtype=work) @ np.asarray(w_router, dtype=work).T).astype(np.float64)
    if router_bias is not None:
        l = l + np.asarray(router_bias, dtype=np.float64)[None, :]
    return l


# ---------------------------------------------------------------------------
# Stage 2: scoring and group-limited top-k
# ---------------------------------------------------------------------------

def _order_desc(v):
    """Indices of v by descending value, equal values by ascending index."""
    return np.argsort(-v, kind="stable")


def route(cfg, logits, score_bias=None):
    """Per-token expert ids [T, k] (int32) and gates [T, k] (float32).

    logits: float32 [T, E] (the comparison tests pass the GPU's own logits).
    """
    logits = np.asarray(logits, dtype=F32)
    T, E = logits.shape
    k, G, Gk = cfg.top_k, cfg.n_group, cfg.topk_group
    assert np.all(np.isfinite(logits)), "logits must be finite"
    if cfg.score_fn == "sigmoid":
        score = sigmoid_f32(logits)
    elif cfg.score_fn == "softmax":
        score = logits
    else:
        raise ValueError(cfg.score_fn)
    sel = score if score_bias is None else (score + np.asarray(score_bias, dtype=F32)[None, :]).astype(F32)
    gs = E // G
    ids = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=F32)
    for t in range(T):
        v = sel[t]
        allowed = np.ones(E, dtype=bool)
        if Gk < G:
            gscore = np.empty(G, dtype=F32)
            for g in range(G):
                top2 = v[g * gs:(g + 1) * gs][_order_desc(v[g * gs:(g + 1) * gs])[:2]]
                gscore[g] = F32(top2[0] + top2[1]) if gs >= 2 else top2[0]
            keep = _order_desc(gscore)[:Gk]
            allowed[:] = False
            for g in keep:
                allowed[g * gs:(g + 1) * gs] = True
        cand = np.flatnonzero(allowed)
        chosen = cand[_order_desc(v[cand])[:k]]
        ids[t] = chosen
        w[t] = _gates(cfg, logits[t], score[t], chosen)
    return ids, w


def _gates(cfg, lrow, srow, chosen):
    one = F32(1.0)
    gamma = F32(cfg.routed_scale)
    if cfg.score_fn == "sigmoid":
        s = srow[chosen]
        if cfg.renormalize:
            tot = F32(0.0)
            for v in s:                       # slot order
                tot = F32(tot + v)
            g = (s / tot).astype(F32)
        else:
            g = s.astype(F32)
    else:
        if cfg.renormalize:
            m = np.max(lrow[chosen])
            e = exp_f32((lrow[chosen] - m).astype(F32))
            tot = F32(0.0)
            for v in e:
                tot = F32(tot + v)
        else:
            m = np.max(lrow)
            e_all = exp_f32((lrow - m).astype(F32))
            tot = F32(0.0)
            for v in e_all:                   # expert-index order
                tot = F32(tot + v)
            e = e_all[chosen]
        g = (e / tot).astype(F32)
    if gamma != one:
        g = (g * gamma).astype(F32)
    return g


# ---------------------------------------------------------------------------
# Stage 3: dispatch (stable permutation into expert-contiguous order)
# ---------------------------------------------------------------------------

def capacity(cfg, T):
    """Per-expert capacity C = ceil(cf * T * k / E), or None without a limit."""
    if cfg.capacity_factor <= 0:
        return None
    return int(math.ceil(float(F32(cfg.capacity_factor)) * T * cfg.top_k / cfg.n_experts))


def dispatch(cfg, ids):
    """Walk pairs p = t*k + j in order; returns dict of int32 arrays:
    raw_counts [E_l], counts [E_l], offsets [E_l+1], perm [R] (row -> p),
    inv [T*k] (p -> row, or -1 for non-local or dropped pairs)."""
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    P = ids.size
    T = P // cfg.top_k
    El, b = cfg.n_local, cfg.expert_begin
    C = capacity(cfg, T)
    raw = [0] * El
    rank = [-1] * P
    for p in range(P):
        le = int(ids[p]) - b
        if 0 <= le < El:
            rank[p] = raw[le]
            raw[le] += 1
    counts = [min(r, C) if C is not None else r for r in raw]
    offsets = [0] * (El + 1)
    for e in range(El):
        offsets[e + 1] = offsets[e] + counts[e]
    R = offsets[El]
    perm = [0] * R
    inv = [-1] * P
    for p in range(P):
        le = int(ids[p]) - b
        if 0 <= le < El and rank[p] < counts[le]:
            row = offsets[le] + rank[p]
            perm[row] = p
            inv[p] = row
    i32 = lambda a: np.asarray(a, dtype=np.int32)
    return dict(raw_counts=i32(raw), counts=i32(counts), offsets=i32(offsets),
                perm=i32(perm), inv=i32(inv))


# ---------------------------------------------------------------------------
# Stage 4: experts (SwiGLU FFN)
# ---------------------------------------------------------------------------

def _round_act(v, act):
    if act == "f32":
        return np.asarray(v, dtype=F32).astype(np.float64)
    if act == "bf16":
        return bf16_round(v)
    raise ValueError(act)


def silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(cfg, x_rows, w13, w2, inter, w13_scale=None, w2_scale=None, round_out=True, work=np.float64):
    """o = (silu(x W_g^T) * (x W_u^T)) W_d^T for the given rows.

    x_rows: [n, H] input rows (their exact stored values). w13: [2I, H] with
    rows 0..I-1 the gate and I..2I-1 the up projection; w2: [H, I]. For fp8
    the weights are e4m3 codes with 128x128 block scales and the activations
    are quantised per 1x128 block before each GEMM; for mxfp4 the weights are
    packed E2M1 codes with E8M0 scales per 32 along the input dimension and
    the activations are MX e4m3 (32-element power-of-two scales). Returns fp64 [n, H]; with
    round_out (routed experts, whose outputs travel through the combine) the
    rows are rounded to their bf16 carrier when activations are bf16 or fp8.
    `work` is the matmuls' arithmetic type: fp64 for every parity use; the CPU
    baseline timing alone passes float32.
    """
    if cfg.act == "fp8":
        W13 = dequant_block_weight(w13, w13_scale)
        W2 = dequant_block_weight(w2, w2_scale)
        qx, sx = quantize_fp8_rows(np.asarray(x_rows, dtype=F32))
        xa = (qx.reshape(len(qx), -1, 128) * sx.astype(np.float64)[:, :, None]).reshape(qx.shape)
    elif cfg.act == "mxfp4":
        W13 = dequant_mx_weight(w13, w13_scale)
        W2 = dequant_mx_weight(w2, w2_scale)
        xa = dequant_mx_rows(*quantize_mx_rows(np.asarray(x_rows, dtype=F32)))
    else:
        W13 = np.asarray(w13, dtype=work)
        W2 = np.asarray(w2, dtype=work)
        xa = np.asarray(x_rows, dtype=work)
    W13, W2, xa = W13.astype(work, copy=False), W2.astype(work, copy=False), xa.astype(work, copy=False)
    g = (xa @ W13[:inter].T).astype(np.float64)
    u = (xa @ W13[inter:].T).astype(np.float64)
    h = silu(g) * u
    if cfg.act == "fp8":
        qh, sh = quantize_fp8_rows(h.astype(F32))
        ha = (qh.reshape(len(qh), -1, 128) * sh.astype(np.float64)[:, :, None]).reshape(qh.shape)
    elif cfg.act == "mxfp4":
        ha = dequant_mx_rows(*quantize_mx_rows(h.astype(F32)))
    else:
        ha = _round_act(h, cfg.act)
    o = (ha.astype(work, copy=False) @ W2.T).astype(np.float64)
    if round_out and cfg.act in ("bf16", "fp8", "mxfp4"):
        o = bf16_round(o)
    return o


# ---------------------------------------------------------------------------
# Stage 5: combine
# ---------------------------------------------------------------------------

def combine(cfg, T, out_rows, inv, w, shared=None):
    """y_t = shared_t + sum_j [inv[t,j] >= 0] * w[t,j] * o[inv[t,j]] (fp64)."""
    H = out_rows.shape[1] if len(out_rows) else cfg.hidden
    k = cfg.top_k
    y = np.zeros((T, H), dtype=np.float64) if shared is None else np.array(shared, dtype=np.float64)
    inv = np.asarray(inv).reshape(T, k)
    w = np.asarray(w, dtype=np.float64).reshape(T, k)
    for t in range(T):
        for j in range(k):
            r = inv[t, j]
            if r >= 0:
                y[t] += w[t, j] * out_rows[r]
    return y


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------

def experts_forward(cfg, x, disp, w13, w2, w13_scale=None, w2_scale=None, work=np.float64):
    """Expert output rows [R, H] in dispatch order (one expert at a time)."""
    x = np.asarray(x)
    k = cfg.top_k
    R = int(disp["offsets"][-1])
    out = np.zeros((R, cfg.hidden), dtype=np.float64)
    for le in range(cfg.n_local):
        a, b = int(disp["offsets"][le]), int(disp["offsets"][le + 1])
        if a == b:
            continue
        tok = disp["perm"][a:b] // k
        out[a:b] = swiglu_expert(cfg, x[tok], w13[le], w2[le], cfg.inter,
                                 None if w13_scale is None else w13_scale[le],
                                 None if w2_scale is None else w2_scale[le], work=work)
    return out


def shared_forward(cfg, x, sw13, sw2, sw13_scale=None, sw2_scale=None, work=np.float64):
    if cfg.shared_inter <= 0:
        return None
    # The shared expert's output stays on the token's own GPU: no bf16 carrier.
    return swiglu_expert(cfg, x, sw13, sw2, cfg.shared_inter, sw13_scale, sw2_scale, round_out=False, work=work)


def forward(cfg, x, w_router, w13, w2, router_bias=None, score_bias=None,
            shared_w13=None, shared_w2=None, logits=None, scales=None, work=np.float64):
    """The whole layer. If `logits` (float32 [T, E]) is given it is used for
    routing instead of the oracle's own router GEMM. `scales` holds the fp8
    block scales dict (w13_scale, w2_scale, shared_w13_scale, shared_w2_scale).
    `work`: the matmuls' arithmetic type (fp64 for parity; float32 only for
    the CPU baseline timing). Returns dict with y (fp64 [T, H]) and every
    intermediate."""
    scales = scales or {}
    x = np.asarray(x)
    T = x.shape[0]
    own_logits = router_logits(x, w_router, router_bias, work=work)
    l32 = own_logits.astype(F32) if logits is None else np.asarray(logits, dtype=F32)
    ids, w = route(cfg, l32, score_bias)
    disp = dispatch(cfg, ids)
    rows = experts_forward(cfg, x, disp, w13, w2, scales.get("w13_scale"), scales.get("w2_scale"), work=work)
    sh = shared_forward(cfg, x, shared_w13, shared_w2,
                        scales.get("shared_w13_scale"), scales.get("shared_w2_scale"), work=work)
    y = combine(cfg, T, rows, disp["inv"], w, sh)
    return dict(y=y, logits=own_logits, ids=ids, w=w, rows=rows, shared=sh, **disp)


def forward_tokens(cfg, tokens, x_rows, ids, w, inv, get_expert, shared_w=None):
    """y for a sample of tokens, given the whole batch's routing.

    tokens: the sampled token indices; x_rows: their hidden states [n, H];
    ids, w, inv: routing of the whole batch (inv from dispatch, so capacity
    drops are those of the whole batch); get_expert(le) -> (w13, w2, w13_scale,
    w2_scale) for local expert le; shared_w: the same tuple for the shared
    expert, or None. Returns fp64 [n, H].
    """
    k = cfg.top_k
    x_rows = np.asarray(x_rows)
    n = len(tokens)
    y = np.zeros((n, cfg.hidden), dtype=np.float64)
    if shared_w is not None:
        y += swiglu_expert(cfg, x_rows, shared_w[0], shared_w[1], cfg.shared_inter, shared_w[2], shared_w[3],
                           round_out=False)
    need = {}
    for i, t in enumerate(tokens):
        for j in range(k):
            if inv[t * k + j] >= 0:
                need.setdefault(int(ids[t, j]) - cfg.expert_begin, []).append((i, j, t))
    for le in sorted(need):
        w13, w2, s13, s2 = get_expert(le)
        idx = [i for i, _, _ in need[le]]
        o = swiglu_expert(cfg, x_rows[idx], w13, w2, cfg.inter, s13, s2)
        for (i, j, t), orow in zip(need[le], o):
            y[i] += float(w[t, j]) * orow
    return y


def rel_max_err(y, y_ref):
    """max |y - y_ref| / RMS(y_ref), the layer-output parity measure."""
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = math.sqrt(float(np.mean(y_ref * y_ref)))
    return float(np.max(np.abs(np.asarray(y, dtype=np.float64) - y_ref))) / rms
