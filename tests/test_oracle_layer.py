"""Pins of the oracle's expert FFN, combine and whole-layer forward.

References: torch's F.silu / F.linear / softmax as library routines, a
brute-force dense evaluation (every expert on every token, masked by the
routing), the expert-parallel share identity, and torch's bf16 / float8 casts
for the carrier-type roundings.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O
from synth import make_inputs, workload

F64 = torch.float64


def _tiny(**kw):
    w = dict(T=48, hidden=128, n_experts=8, expert_begin=0, expert_end=8, top_k=2,
             n_group=1, topk_group=1, score_fn="softmax", renormalize=True,
             routed_scale=1.0, inter=128, shared_inter=0, dtype="f32",
             capacity_factor=0.0, score_bias="none", router_bias="none")
    w.update(kw)
    return w


def _np(t):
    return None if t is None else t.float().numpy() if t.dtype != torch.float8_e4m3fn else t.view(torch.uint8).numpy()


def _torch_swiglu(x, w13, w2, I):
    x = torch.as_tensor(x, dtype=F64)
    w13 = torch.as_tensor(w13, dtype=F64)
    w2 = torch.as_tensor(w2, dtype=F64)
    return F.linear(F.silu(F.linear(x, w13[:I])) * F.linear(x, w13[I:]), w2)


def test_single_expert_top1_is_plain_swiglu_mlp():
    w = _tiny(n_experts=1, expert_end=1, top_k=1)
    inp = make_inputs(w)
    cfg = O.Config.from_workload(w)
    out = O.forward(cfg, _np(inp["x"]), _np(inp["w_router"]), _np(inp["w13"]), _np(inp["w2"]))
    ref = _torch_swiglu(_np(inp["x"]), _np(inp["w13"])[0], _np(inp["w2"])[0], w["inter"]).numpy()
    assert np.all(out["w"] == 1.0)
    # the oracle rounds h to float32 for fp32 activations (relative 2**-24)
    assert O.rel_max_err(out["y"], ref) < 1e-6


def _dense_reference(cfg, x, ids, w, inv, w13, w2, shared=None):
    """Every expert on every token, then a dense [T, E_l] gate mask."""
    T = x.shape[0]
    k = cfg.top_k
    gate = np.zeros((T, cfg.n_local))
    for t in range(T):
        for j in range(k):
            if inv[t * k + j] >= 0:
                gate[t, ids[t, j] - cfg.expert_begin] += w[t, j]
    y = np.zeros((T, cfg.hidden)) if shared is None else shared.copy()
    for e in range(cfg.n_local):
        y += gate[:, e:e + 1] * _torch_swiglu(x, w13[e], w2[e], cfg.inter).numpy()
    return y


@pytest.mark.parametrize("kw", [
    dict(),
    dict(top_k=3, n_group=4, topk_group=2, score_fn="sigmoid", score_bias="normal0.1"),
    dict(expert_begin=2, expert_end=6, top_k=3, score_fn="sigmoid"),
    dict(top_k=2, capacity_factor=1.0),
    dict(shared_inter=128, top_k=2, score_fn="sigmoid", routed_scale=2.5),
])
def test_sparse_oracle_matches_dense_brute_force(kw):
    w = _tiny(**kw)
    inp = make_inputs(w)
    cfg = O.Config.from_workload(w)
    x = _np(inp["x"])
    out = O.forward(cfg, x, _np(inp["w_router"]), _np(inp["w13"]), _np(inp["w2"]),
                    score_bias=_np(inp["score_bias"]), shared_w13=_np(inp["shared_w13"]),
                    shared_w2=_np(inp["shared_w2"]))
    sh = None
    if cfg.shared_inter:
        sh = _torch_swiglu(x, _np(inp["shared_w13"]), _np(inp["shared_w2"]), cfg.shared_inter).numpy()
    ref = _dense_reference(cfg, x, out["ids"], out["w"], out["inv"], _np(inp["w13"]), _np(inp["w2"]), sh)
    assert O.rel_max_err(out["y"], ref) < 1e-6


def test_softmax_all_experts_is_dense_softmax_mixture():
    w = _tiny(top_k=8, renormalize=False)
    inp = make_inputs(w)
    cfg = O.Config.from_workload(w)
    x, wr = _np(inp["x"]), _np(inp["w_router"])
    out = O.forward(cfg, x, wr, _np(inp["w13"]), _np(inp["w2"]))
    p = torch.softmax(torch.from_numpy(x).double() @ torch.from_numpy(wr).double().T, -1).numpy()
    ref = sum(p[:, e:e + 1] * _torch_swiglu(x, _np(inp["w13"])[e], _np(inp["w2"])[e], cfg.inter).numpy()
              for e in range(8))
    assert O.rel_max_err(out["y"], ref) < 1e-6


def test_expert_parallel_shares_sum_to_whole_layer():
    """Each GPU holds 256/EP routed experts plus a replica of the shared expert
    (Perplexity, 'Expert parallelism'); the partial outputs of the EP shares,
    less the extra shared copies, add up to the whole layer."""
    full = _tiny(n_experts=16, expert_end=16, top_k=4, n_group=4, topk_group=2,
                 score_fn="sigmoid", score_bias="normal0.1", shared_inter=128)
    EP = 4
    inp = make_inputs(full)
    cfg = O.Config.from_workload(full)
    args = lambda inp: (_np(inp["x"]), _np(inp["w_router"]), _np(inp["w13"]), _np(inp["w2"]))
    kw = lambda inp: dict(score_bias=_np(inp["score_bias"]), shared_w13=_np(inp["shared_w13"]),
                          shared_w2=_np(inp["shared_w2"]))
    y_full = O.forward(cfg, *args(inp), **kw(inp))["y"]
    acc = None
    for r in range(EP):
        wr = dict(full, expert_begin=4 * r, expert_end=4 * r + 4)
        ir = make_inputs(wr)          # same seeds: experts 4r..4r+3 of the full layer
        assert torch.equal(ir["w13"], inp["w13"][4 * r:4 * r + 4])
        yr = O.forward(O.Config.from_workload(wr), *args(ir), **kw(ir))["y"]
        acc = yr if acc is None else acc + yr
    sh = O.forward(cfg, *args(inp), **kw(inp))["shared"]
    np.testing.assert_allclose(acc - (EP - 1) * sh, y_full, rtol=0, atol=1e-12)


def _equal_up_to_rare_flips(got, ref):
    """Equal, except where the two fp64 matmuls (different summation orders)
    land on opposite sides of a rounding boundary: one bf16 step at most."""
    assert np.mean(got == ref) > 0.99
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30)


def test_bf16_carrier_roundings_match_torch():
    w = _tiny(dtype="bf16", shared_inter=128, score_fn="sigmoid")
    inp = make_inputs(w)
    cfg = O.Config.from_workload(w)
    x = inp["x"].double()
    w13, w2 = inp["w13"][3].double(), inp["w2"][3].double()
    got = O.swiglu_expert(cfg, _np(inp["x"]), _np(inp["w13"])[3], _np(inp["w2"])[3], 128)
    h = (F.silu(F.linear(x, w13[:128])) * F.linear(x, w13[128:]))
    # torch's fp64 -> bf16 cast is a single round-to-nearest-even
    h = h.to(torch.bfloat16).double()
    ref = F.linear(h, w2).to(torch.bfloat16).double().numpy()
    _equal_up_to_rare_flips(got, ref)


def test_fp8_block_path_matches_torch_casts():
    w = _tiny(dtype="fp8", T=16, hidden=256, inter=256)
    inp = make_inputs(w)
    cfg = O.Config.from_workload(w)
    e = 5
    got = O.swiglu_expert(cfg, _np(inp["x"]), _np(inp["w13"])[e], _np(inp["w2"])[e], 256,
                          _np(inp["w13_scale"])[e], _np(inp["w2_scale"])[e])

    def deq_w(q, s):
        return q.double() * s.double().repeat_interleave(128, 0).repeat_interleave(128, 1)

    def quant_act(v):           # float32 v [n, K] -> dequantised float64 values
        b = v.reshape(v.shape[0], -1, 128)
        a = b.abs().amax(-1, keepdim=True)
        # (a scalar divided by a tensor is a reciprocal times the scalar in
        # torch, which rounds twice; divide two tensors instead)
        inv = torch.where(a > 0, torch.full_like(a, 448.0) / a, torch.ones_like(a))
        q = (b * inv).to(torch.float8_e4m3fn).double()
        s = torch.where(a > 0, a / torch.full_like(a, 448.0), torch.ones_like(a)).double()
        return (q * s).reshape(v.shape)

    W13 = deq_w(inp["w13"][e], inp["w13_scale"][e])
    W2 = deq_w(inp["w2"][e], inp["w2_scale"][e])
    xa = quant_act(inp["x"].float())
    h = F.silu(F.linear(xa, W13[:256])) * F.linear(xa, W13[256:])
    ha = quant_act(h.float())
    ref = F.linear(ha, W2).to(torch.bfloat16).double().numpy()
    _equal_up_to_rare_flips(got, ref)


def test_toy_workload_routes_like_softmax_top2():
    w = workload("toy_fp32", T=256)
    inp = make_inputs(w)
    cfg = O.Config.from_workload(w)
    out = O.forward(cfg, _np(inp["x"]), _np(inp["w_router"]), _np(inp["w13"]), _np(inp["w2"]))
    l = torch.from_numpy(_np(inp["x"])).double() @ torch.from_numpy(_np(inp["w_router"])).double().T
    assert np.array_equal(out["ids"], torch.topk(l.float(), 2, -1).indices.numpy())
    assert out["counts"].sum() == 512
