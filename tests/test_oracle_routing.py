"""Pins of the oracle's router (scores, group-limited top-k, gates).

Pins: the Ultralytics glossary's worked routing example (printed count ranges),
torch.topk / torch.softmax on special cases that reduce to them, a brute-force
subset enumeration of group-limited selection, and a hand-derived case where
the group rule matters.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

F32 = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cfg(**kw):
    base = dict(hidden=8, n_experts=8, top_k=2, inter=8)
    base.update(kw)
    return O.Config(**base)


def _p3_logits():
    g = json.load(open(os.path.join(GOLDEN, "p3_routing_counts.json")))
    s = g["setup"]
    torch.manual_seed(s["torch_seed"])
    tokens = torch.randn(*s["tokens"])
    router = torch.nn.Linear(s["tokens"][1], s["num_experts"])
    with torch.no_grad():
        logits = router(tokens)
    return g, logits


def test_p3_worked_example_counts():
    """Glossary 'Expert Parallelism' routing snippet: per-expert counts span
    948..1087 of 8192 assignments, per-GPU counts 1968..2139."""
    g, logits = _p3_logits()
    p = g["printed"]
    cfg = _cfg(hidden=512, top_k=2, score_fn="softmax")
    ids, w = O.route(cfg, logits.numpy())
    d = O.dispatch(cfg, ids)
    counts = d["counts"]
    assert counts.sum() == p["assignments"]
    assert counts.min() == p["per_expert_min"] and counts.max() == p["per_expert_max"]
    per_gpu = counts.reshape(4, 2).sum(axis=1)
    assert per_gpu.min() == p["per_gpu_min"] and per_gpu.max() == p["per_gpu_max"]


def test_p3_softmax_top2_equals_torch_topk():
    _, logits = _p3_logits()
    cfg = _cfg(hidden=512, top_k=2, score_fn="softmax")
    ids, w = O.route(cfg, logits.numpy())
    _, ref = torch.softmax(logits, -1).topk(2, dim=-1)
    assert np.array_equal(ids, ref.numpy())
    # renormalised gates: softmax restricted to the two selected experts
    pr = torch.softmax(logits.double(), -1).gather(1, ref)
    pr = (pr / pr.sum(-1, keepdim=True)).numpy()
    np.testing.assert_allclose(w, pr, rtol=1e-6, atol=0)


def test_softmax_all_experts_no_renorm_is_dense_softmax():
    rng = np.random.default_rng(0)
    logits = (rng.standard_normal((64, 16)) * 3).astype(F32)
    cfg = _cfg(n_experts=16, top_k=16, score_fn="softmax", renormalize=False)
    ids, w = O.route(cfg, logits)
    dense = torch.softmax(torch.from_numpy(logits).double(), -1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(dense, ids, 1), rtol=1e-6)
    assert np.array_equal(np.sort(ids, 1), np.tile(np.arange(16), (64, 1)))


def test_all_groups_kept_equals_ungrouped_topk():
    """Mixtral routing is DeepSeek routing with every group kept (Perplexity,
    'MoE Router')."""
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((200, 64)).astype(F32)
    bias = (rng.standard_normal(64) * 0.1).astype(F32)
    a = O.route(_cfg(n_experts=64, top_k=6, n_group=8, topk_group=8, score_fn="sigmoid"), logits, bias)
    b = O.route(_cfg(n_experts=64, top_k=6, n_group=1, topk_group=1, score_fn="sigmoid"), logits, bias)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    sel = O.sigmoid_f32(logits) + bias
    _, ref = torch.from_numpy(sel).topk(6, dim=-1)
    assert np.array_equal(a[0], ref.numpy())


def test_group_rule_hand_case():
    """Groups of two; the group score is the sum of its two best experts, so
    group 1 (3.0 + 2.9) and group 3 (4.0 + 1.5) win over group 0 (5.0 + 0.0),
    although group 0 holds the single best expert."""
    l = np.array([[5.0, 0.0, 3.0, 2.9, 2.0, 2.0, 4.0, 1.5]], dtype=F32)
    ids, w = O.route(_cfg(n_group=4, topk_group=2, top_k=2, score_fn="softmax"), l)
    assert ids.tolist() == [[6, 2]]
    ids, _ = O.route(_cfg(n_group=1, topk_group=1, top_k=2, score_fn="softmax"), l)
    assert ids.tolist() == [[0, 6]]


def test_ties_go_to_lower_index():
    l = np.array([[1.0, 2.0, 2.0, 1.0, 2.0, 2.0, 0.0, 0.0]], dtype=F32)
    ids, _ = O.route(_cfg(top_k=3, score_fn="softmax"), l)
    assert ids.tolist() == [[1, 2, 4]]
    # groups of two: group 2 scores 4.0, groups 0 and 1 tie at 3.0 -> keep 2, 0
    ids, _ = O.route(_cfg(n_group=4, topk_group=2, top_k=2, score_fn="softmax"), l)
    assert ids.tolist() == [[1, 4]]
    # groups 0, 1, 2 all score 3.0: keep the two lowest, 0 and 1
    l2 = np.array([[1.0, 2.0, 2.0, 1.0, 1.5, 1.5, 0.0, 0.0]], dtype=F32)
    ids, _ = O.route(_cfg(n_group=4, topk_group=2, top_k=2, score_fn="softmax"), l2)
    assert ids.tolist() == [[1, 2]]
    # -0 and +0 compare equal
    z = np.array([[-0.0, 0.0, -1.0, -1.0, -1.0, -1.0, -1.0, -1.0]], dtype=F32)
    ids, _ = O.route(_cfg(top_k=2, score_fn="softmax"), z)
    assert ids.tolist() == [[0, 1]]


def _brute_select(v, G, Gk, k):
    """Group-limited top-k by subset enumeration (tiny E only)."""
    E = len(v)
    gs = E // G
    gscore = []
    for g in range(G):
        m = v[g * gs:(g + 1) * gs]
        gscore.append(max(F32(m[i] + m[j]) for i in range(gs) for j in range(gs) if i != j))
    best = None
    for S in itertools.combinations(range(G), Gk):
        key = (sorted([gscore[g] for g in S], reverse=True), [-g for g in S])
        if best is None or key > best[0]:
            best = (key, S)
    allowed = [e for g in best[1] for e in range(g * gs, (g + 1) * gs)]
    bestk = None
    for S in itertools.combinations(allowed, k):
        key = (sorted([v[e] for e in S], reverse=True), [-e for e in S])
        if bestk is None or key > bestk[0]:
            bestk = (key, S)
    return sorted(bestk[1], key=lambda e: (-v[e], e))


@pytest.mark.parametrize("E,G,Gk,k", [(8, 4, 2, 2), (12, 4, 2, 3), (16, 4, 3, 4), (8, 2, 1, 3)])
def test_group_limited_matches_subset_enumeration(E, G, Gk, k):
    rng = np.random.default_rng(E * 100 + G * 10 + k)
    # coarse values so that exact ties are common
    logits = (rng.integers(-6, 6, (60, E)) * 0.5).astype(F32)
    bias = (rng.integers(-2, 3, E) * 0.25).astype(F32)
    cfg = _cfg(n_experts=E, top_k=k, n_group=G, topk_group=Gk, score_fn="sigmoid")
    ids, w = O.route(cfg, logits, bias)
    sel = (O.sigmoid_f32(logits) + bias).astype(F32)
    for t in range(len(logits)):
        assert ids[t].tolist() == _brute_select(sel[t], G, Gk, k)


def test_sigmoid_gates_use_unbiased_score_and_sum_to_scale():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((300, 32)).astype(F32)
    bias = (rng.standard_normal(32) * 2.0).astype(F32)    # large: flips choices
    for gamma in (1.0, 2.5):
        cfg = _cfg(n_experts=32, top_k=4, n_group=4, topk_group=2, score_fn="sigmoid", routed_scale=gamma)
        ids, w = O.route(cfg, logits, bias)
        s = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
        ref = np.take_along_axis(s, ids, 1)
        ref = gamma * ref / ref.sum(1, keepdims=True)
        np.testing.assert_allclose(w, ref, rtol=4e-7)
        np.testing.assert_allclose(w.sum(1), gamma, rtol=1e-6)
    # the bias changed the selection relative to the unbiased top-k
    ids_nb, _ = O.route(cfg, logits, None)
    assert not np.array_equal(ids, ids_nb)


def test_route_invariants_deepseek_shape():
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((64, 256)).astype(F32)
    bias = (rng.standard_normal(256) * 0.1).astype(F32)
    cfg = _cfg(n_experts=256, top_k=8, n_group=8, topk_group=4, score_fn="sigmoid")
    ids, w = O.route(cfg, logits, bias)
    for t in range(64):
        assert len(set(ids[t].tolist())) == 8
        assert len(set((ids[t] // 32).tolist())) <= 4
    assert np.all(w > 0)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-6)
