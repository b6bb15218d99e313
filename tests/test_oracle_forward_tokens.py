"""Pins of the oracle functions the full-size GPU parity tests lean on:
forward_tokens (the layer output of a sample of tokens, given the whole
batch's routing) and router_logits with the router's linear bias.

forward_tokens is pinned two ways, on tiny layers with capacity drops, a
local expert share, a shared expert, the Zipf router bias and the fp8 path:
  * against the whole-layer oracle, O.forward()['y'] restricted to the sample;
  * against a dense brute force (every local expert on every token, masked by
    a dense gate matrix built from the routing, plus the shared expert through
    torch's F.linear / F.silu), for every token and for a random subset.
router_logits with a bias is pinned against torch's F.linear(x, W, c).

Each pin is shown to catch the mistakes it exists for: a copy of the oracle
function with one planted mistake (gate of the sample index instead of the
token, capacity drops ignored, the shared expert added twice, the bias
subtracted or added along the wrong axis) must fail it.
"""
import inspect
import textwrap

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O
from synth import make_inputs

F64 = torch.float64


def _np(t):
    if t is None:
        return None
    return t.view(torch.uint8).numpy() if t.dtype == torch.float8_e4m3fn else t.float().numpy()


def _tiny(**kw):
    w = dict(T=64, hidden=128, n_experts=16, expert_begin=0, expert_end=16, top_k=4, n_group=4, topk_group=2,
             score_fn="sigmoid", renormalize=True, routed_scale=1.0, inter=128, shared_inter=128, dtype="f32",
             capacity_factor=0.0, score_bias="normal0.1", router_bias="none")
    w.update(kw)
    return w


# Layers whose routing exercises what forward_tokens must get right.
CASES = {
    # capacity 1.0 with the Zipf router bias: many pairs dropped
    "capacity_zipf_shared": dict(capacity_factor=1.0, router_bias="zipf1.1"),
    # a local share: pairs of other experts are non-local (inv = -1)
    "share_capacity": dict(expert_begin=4, expert_end=11, capacity_factor=1.5),
    # no shared expert, softmax routing, gates without renormalisation
    "softmax_no_shared": dict(score_fn="softmax", n_group=1, topk_group=1, top_k=3, shared_inter=0,
                              renormalize=False, score_bias="none", routed_scale=2.5),
    # bf16 carriers (h and the routed rows rounded)
    "bf16_share_capacity": dict(dtype="bf16", expert_begin=2, expert_end=14, capacity_factor=1.25,
                                router_bias="zipf1.1"),
    # e4m3 weights and activations with block scales
    "fp8_capacity_zipf": dict(dtype="fp8", capacity_factor=1.25, router_bias="zipf1.1", score_bias="zero",
                              T=48),
}


def _layer(w):
    inp = make_inputs(w)
    cfg = O.Config.from_workload(w)
    h = {k: _np(v) for k, v in inp.items()}
    scales = {k: h.get(k) for k in ("w13_scale", "w2_scale", "shared_w13_scale", "shared_w2_scale")}
    out = O.forward(cfg, h["x"], h["w_router"], h["w13"], h["w2"], router_bias=h["router_bias"],
                    score_bias=h["score_bias"], shared_w13=h.get("shared_w13"), shared_w2=h.get("shared_w2"),
                    scales=scales)
    return cfg, h, out


def _sample_y(fn, cfg, h, out, tokens):
    def get_expert(le):
        s13 = h["w13_scale"][le] if h.get("w13_scale") is not None else None
        s2 = h["w2_scale"][le] if h.get("w2_scale") is not None else None
        return h["w13"][le], h["w2"][le], s13, s2

    sh = None
    if cfg.shared_inter:
        sh = (h["shared_w13"], h["shared_w2"], h.get("shared_w13_scale"), h.get("shared_w2_scale"))
    return fn(cfg, tokens, h["x"][tokens], out["ids"], out["w"], out["inv"], get_expert, sh)


def _samples(cfg, out, T, rng):
    """A random subset that contains a token that lost a pair to capacity (if
    any), a token with a non-local pair (if any) and tokens whose sample index
    differs from their token index; and every token."""
    inv = out["inv"].reshape(T, cfg.top_k)
    local = (out["ids"] >= cfg.expert_begin) & (out["ids"] < cfg.expert_end)
    dropped = np.nonzero(((inv < 0) & local).any(axis=1))[0]
    nonlocal_ = np.nonzero((~local).any(axis=1))[0]
    sub = set(rng.choice(T, min(9, T), replace=False).tolist())
    if len(dropped):
        sub.add(int(dropped[-1]))
    if len(nonlocal_):
        sub.add(int(nonlocal_[0]))
    return [sorted(sub, reverse=True), list(range(T))]


@pytest.mark.parametrize("name", list(CASES))
def test_forward_tokens_equals_whole_layer(name):
    w = _tiny(**CASES[name])
    cfg, h, out = _layer(w)
    rng = np.random.default_rng(5)
    for tok in _samples(cfg, out, w["T"], rng):
        got = _sample_y(O.forward_tokens, cfg, h, out, tok)
        want = out["y"][tok]
        scale = float(np.sqrt(np.mean(out["y"] ** 2)))
        # the two sum the same fp64 terms in different orders
        assert np.max(np.abs(got - want)) <= 1e-12 * scale


def _dense(cfg, h, out):
    """Every local expert on every token (torch F.linear / F.silu in fp64),
    masked by a dense [T, E_l] gate matrix, plus the shared expert. fp32 only:
    the carriers of bf16 and fp8 are pinned elsewhere."""
    T = h["x"].shape[0]
    x = torch.from_numpy(h["x"]).to(F64)
    gate = np.zeros((T, cfg.n_local))
    inv = out["inv"].reshape(T, cfg.top_k)
    for t in range(T):
        for j in range(cfg.top_k):
            if inv[t, j] >= 0:
                gate[t, out["ids"][t, j] - cfg.expert_begin] += out["w"][t, j]

    def mlp(w13, w2, I):
        w13 = torch.from_numpy(np.asarray(w13)).to(F64)
        w2 = torch.from_numpy(np.asarray(w2)).to(F64)
        return F.linear(F.silu(F.linear(x, w13[:I])) * F.linear(x, w13[I:]), w2).numpy()

    y = np.zeros((T, cfg.hidden))
    if cfg.shared_inter:
        y += mlp(h["shared_w13"], h["shared_w2"], cfg.shared_inter)
    for e in range(cfg.n_local):
        y += gate[:, e:e + 1] * mlp(h["w13"][e], h["w2"][e], cfg.inter)
    return y


@pytest.mark.parametrize("name", [n for n in CASES if CASES[n].get("dtype", "f32") == "f32"])
def test_forward_tokens_equals_dense_brute_force(name):
    w = _tiny(**CASES[name])
    cfg, h, out = _layer(w)
    ref = _dense(cfg, h, out)
    rng = np.random.default_rng(9)
    for tok in _samples(cfg, out, w["T"], rng):
        got = _sample_y(O.forward_tokens, cfg, h, out, tok)
        # the oracle rounds h to float32 for fp32 activations (relative 2**-24)
        assert O.rel_max_err(got, ref[tok]) < 1e-6


def test_samples_exercise_drops_shares_and_reindexing():
    """The layers above really contain what the pins rely on."""
    cfg, h, out = _layer(_tiny(**CASES["capacity_zipf_shared"]))
    assert int((out["raw_counts"] - out["counts"]).sum()) > 0
    cfg, h, out = _layer(_tiny(**CASES["share_capacity"]))
    assert np.any(out["inv"] < 0) and int((out["raw_counts"] - out["counts"]).sum()) > 0
    cfg, h, out = _layer(_tiny(**CASES["fp8_capacity_zipf"]))
    assert int((out["raw_counts"] - out["counts"]).sum()) > 0


def _mutant(fn, old, new):
    """A copy of oracle function `fn` with `old` replaced by `new` in its source."""
    src = textwrap.dedent(inspect.getsource(fn))
    assert old in src, old
    ns = dict(vars(O))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns[fn.__name__]


MUTANTS = [
    ("float(w[t, j])", "float(w[i, j])"),                        # gate of the sample index
    ("if inv[t * k + j] >= 0:", "if int(ids[t, j]) - cfg.expert_begin in range(cfg.n_local):"),  # no drops
    ("y += swiglu_expert(", "y += 2 * swiglu_expert("),          # shared expert twice
    ("for le in sorted(need):", "for le in sorted(need)[1:]:"),  # an expert left out
]


@pytest.mark.parametrize("old,new", MUTANTS, ids=["gate_index", "no_drops", "shared_twice", "expert_missing"])
def test_planted_forward_tokens_mistakes_are_caught(old, new):
    bad = _mutant(O.forward_tokens, old, new)
    caught = False
    for name in ("capacity_zipf_shared", "share_capacity"):
        cfg, h, out = _layer(_tiny(**CASES[name]))
        for tok in _samples(cfg, out, out["ids"].shape[0], np.random.default_rng(5)):
            got = _sample_y(bad, cfg, h, out, tok)
            scale = float(np.sqrt(np.mean(out["y"] ** 2)))
            caught |= bool(np.max(np.abs(got - out["y"][tok])) > 1e-12 * scale)
    assert caught


# ---------------------------------------------------------------------------
# router_logits with the router's linear bias (the Zipf popularity offset)
# ---------------------------------------------------------------------------

def _router_case(dtype):
    w = _tiny(dtype=dtype, n_experts=256, expert_end=256, n_group=8, top_k=8, hidden=256, T=40,
              router_bias="zipf1.1")
    inp = make_inputs(w)
    return inp


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_router_logits_with_bias_match_linear(dtype):
    inp = _router_case(dtype)
    x, wr, c = _np(inp["x"]), _np(inp["w_router"]), _np(inp["router_bias"])
    assert c is not None and np.ptp(c) > 1.0                     # a real, non-constant offset
    got = O.router_logits(x, wr, c)
    want = F.linear(torch.from_numpy(x).to(F64), torch.from_numpy(wr).to(F64), torch.from_numpy(c).to(F64))
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-13, atol=1e-13)
    # without the bias the logits differ by exactly the broadcast offset
    np.testing.assert_allclose(got - O.router_logits(x, wr), np.broadcast_to(c.astype(np.float64), got.shape),
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("old,new", [
    ("l = l + np.asarray(router_bias", "l = l - np.asarray(router_bias"),
    ("[None, :]", "[:, None][:l.shape[0]]"),
], ids=["bias_sign", "bias_axis"])
def test_planted_router_bias_mistakes_are_caught(old, new):
    inp = _router_case("f32")
    x, wr, c = _np(inp["x"]), _np(inp["w_router"]), _np(inp["router_bias"])
    bad = _mutant(O.router_logits, old, new)
    want = F.linear(torch.from_numpy(x).to(F64), torch.from_numpy(wr).to(F64), torch.from_numpy(c).to(F64))
    try:
        got = bad(x, wr, c)
    except ValueError:
        return                                                   # a shape error is caught too
    assert not np.allclose(got, want.numpy(), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_float32_work_type_stays_within_tolerance(dtype):
    """The CPU baseline times the oracle with float32 matmuls; that variant
    routes identically and stays well within the layer tolerance of the fp64
    oracle (it is never used for parity)."""
    w = _tiny(dtype=dtype, capacity_factor=1.25, router_bias="zipf1.1", score_bias="zero", T=48)
    inp = make_inputs(w)
    cfg = O.Config.from_workload(w)
    h = {k: _np(v) for k, v in inp.items()}
    scales = {k: h.get(k) for k in ("w13_scale", "w2_scale", "shared_w13_scale", "shared_w2_scale")}
    args = (cfg, h["x"], h["w_router"], h["w13"], h["w2"])
    kw = dict(router_bias=h["router_bias"], score_bias=h["score_bias"], shared_w13=h["shared_w13"],
              shared_w2=h["shared_w2"], scales=scales)
    ref = O.forward(*args, **kw)
    got = O.forward(*args, work=np.float32, **kw)
    assert np.array_equal(got["ids"], ref["ids"])
    assert O.rel_max_err(got["y"], ref["y"]) < 0.2 * {"bf16": 2e-2, "fp8": 6e-2}[dtype]
