"""The Ultralytics glossary's worked routing example ("Expert Parallelism",
section "How tokens move between GPUs") through the GPU: 4096 tokens of width
512, a linear router to 8 experts (seed 0), softmax top-2, 8 experts on 4
GPUs. The page prints per-expert counts from 948 to 1087 (8192 assignments,
1024 each if uniform) and per-GPU counts from 1968 to 2139
(tests/golden/p3_routing_counts.json).

Two paths: the snippet's own logits (torch on the CPU) given to moe_route and
moe_dispatch, and the snippet's tokens, router weight and bias given to the
GPU's router GEMM (fp32, with the linear bias) first. The smallest gap
between a token's second and third logit is 2.8e-5, far above the fp32
GEMM's rounding at K = 512, so both paths must give the printed counts.
"""
import json
import os

import numpy as np
import pytest
import torch

import mixture_experts_layer_10_amd as moe
from oracle import moe_oracle as O

from gpu_helpers import host, say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p3_routing_counts.json")


def _snippet():
    g = json.load(open(GOLDEN))
    s = g["setup"]
    torch.manual_seed(s["torch_seed"])
    tokens = torch.randn(*s["tokens"])
    router = torch.nn.Linear(s["tokens"][1], s["num_experts"])
    with torch.no_grad():
        logits = router(tokens)
    return g, tokens, router.weight.detach().clone(), router.bias.detach().clone(), logits


def _route_dispatch(cfg, logits_dev, T):
    ids = torch.empty(T, 2, dtype=torch.int32, device="cuda")
    w = torch.empty(T, 2, dtype=torch.float32, device="cuda")
    moe.moe_route(cfg, logits_dev, None, ids, w)
    d = dict(raw_counts=torch.empty(8, dtype=torch.int32, device="cuda"),
             counts=torch.empty(8, dtype=torch.int32, device="cuda"),
             offsets=torch.empty(9, dtype=torch.int32, device="cuda"),
             perm=torch.empty(T * 2, dtype=torch.int32, device="cuda"),
             inv=torch.empty(T * 2, dtype=torch.int32, device="cuda"))
    moe.moe_dispatch(cfg, ids, d["raw_counts"], d["counts"], d["offsets"], d["perm"], d["inv"], moe.workspace(cfg, T))
    torch.cuda.synchronize()
    return host(ids), host(w), {k: host(v) for k, v in d.items()}


def _check_printed(counts, printed):
    assert int(counts.sum()) == printed["assignments"]
    assert counts.min() == printed["per_expert_min"] and counts.max() == printed["per_expert_max"]
    per_gpu = counts.reshape(4, 2).sum(axis=1)
    assert per_gpu.min() == printed["per_gpu_min"] and per_gpu.max() == printed["per_gpu_max"]


@pytest.mark.parametrize("path", ["snippet_logits", "gpu_router_gemm"])
def test_glossary_routing_example_on_gpu(path):
    g, x, W, b, logits = _snippet()
    T = x.shape[0]
    say("glossary routing example:", path, "T", T)
    cfg = moe.make_config(512, 8, 2, 128, dtype="f32", score_fn="softmax", n_group=1, topk_group=1)
    ocfg = O.Config(hidden=512, n_experts=8, top_k=2, inter=128, score_fn="softmax")
    if path == "snippet_logits":
        l_dev = logits.cuda()
    else:
        l_dev = torch.empty(T, 8, dtype=torch.float32, device="cuda")
        moe.moe_router_gemm(cfg, x.cuda(), W.cuda(), b.cuda(), l_dev, moe.workspace(cfg, T))
        torch.cuda.synchronize()
        want = O.router_logits(x.numpy(), W.numpy(), b.numpy())
        assert O.rel_max_err(host(l_dev), want) < 1e-5
    ids, w, d = _route_dispatch(cfg, l_dev, T)
    # the GPU's routing and dispatch equal the oracle's on the same logits, bit for bit
    oid, ow = O.route(ocfg, host(l_dev))
    od = O.dispatch(ocfg, oid)
    assert np.array_equal(ids, oid) and np.array_equal(w.view(np.int32), ow.view(np.int32))
    for key in ("raw_counts", "counts", "offsets", "inv"):
        assert np.array_equal(d[key], od[key]), key
    assert np.array_equal(d["perm"], od["perm"])
    # and reproduce the page's printed counts
    say("  per-expert counts", d["counts"].tolist())
    _check_printed(d["counts"], g["printed"])
