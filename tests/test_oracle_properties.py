"""Property tests of the oracle's routing and dispatch over random
configurations drawn by hypothesis. Each checks an invariant the method fixes
directly on the outputs, with its own arithmetic (a sort for the group score,
a total order on (score, index), float64 gate formulas), not by re-running the
oracle's steps:

  routing   k distinct experts per token, from at most G_k groups; no kept
            group ranks below a dropped one by group score (the sum of its two
            best selection scores); no allowed expert left out ranks above a
            chosen one; slots in rank order; gates from the unbiased scores,
            summing to the scaling factor when renormalised;
  dispatch  counts are the local pair counts capped at the capacity; offsets
            their exclusive scan; perm and inv inverse bijections between rows
            and kept pairs; rows of an expert in pair order; capacity keeps
            each expert's first pairs.

Pages: NVIDIA "Optimizing DeepSeek R1 throughput on Blackwell", "Top-K kernel
fusion" (groups first, then the top experts inside them); Ultralytics
"Expert Parallelism", "Load balancing and capacity" (selection-only bias,
capacity); Perplexity "Lower latency and higher throughput with multi-node
DeepSeek deployment", "MoE Router" (assignments gathered per expert).
"""
import numpy as np
from hypothesis import HealthCheck, given, settings, strategies as st

from oracle import moe_oracle as O

F32 = np.float32
SETTINGS = dict(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def router_case(draw):
    E = draw(st.sampled_from([4, 8, 16, 32, 64]))
    G = draw(st.sampled_from([g for g in (1, 2, 4, 8) if E % g == 0 and (g == 1 or E // g >= 2)]))
    Gk = draw(st.integers(1, G))
    k = draw(st.integers(1, min(16, Gk * (E // G))))
    T = draw(st.integers(0, 24))
    score_fn = draw(st.sampled_from(["softmax", "sigmoid"]))
    kind = draw(st.sampled_from(["normal", "ties", "wide"]))
    rng = np.random.default_rng(draw(st.integers(0, 2 ** 31 - 1)))
    logits = rng.standard_normal((T, E)).astype(F32)
    if kind == "ties":
        logits = (np.round(logits * 2) / 2).astype(F32)           # many exact ties
    elif kind == "wide":
        logits = (logits * 40).astype(F32)                        # saturated scores
    bias = None
    if score_fn == "sigmoid" and draw(st.booleans()):
        bias = (rng.standard_normal(E) * 0.1).astype(F32)
        if kind == "ties":
            bias = (np.round(bias * 8) / 8).astype(F32)
    cfg = O.Config(hidden=8, n_experts=E, top_k=k, inter=8, n_group=G, topk_group=Gk, score_fn=score_fn,
                   renormalize=draw(st.booleans()), routed_scale=draw(st.sampled_from([1.0, 2.5])))
    return cfg, logits, bias


def _beats(v, i, w, j):
    """(v, i) ranks above (w, j): larger score, or equal score and lower index."""
    return v > w or (v == w and i < j)


@settings(**SETTINGS)
@given(router_case())
def test_route_properties(case):
    cfg, logits, bias = case
    T, E = logits.shape
    k, G, Gk = cfg.top_k, cfg.n_group, cfg.topk_group
    gs = E // G
    ids, w = O.route(cfg, logits, bias)
    assert ids.shape == (T, k) and w.shape == (T, k)
    score = O.sigmoid_f32(logits) if cfg.score_fn == "sigmoid" else logits
    sel = score if bias is None else (score + bias[None, :]).astype(F32)
    for t in range(T):
        row, v = ids[t], sel[t]
        assert len(set(row.tolist())) == k and row.min() >= 0 and row.max() < E
        # groups: the two best selection scores of each group, summed in fp32
        if Gk < G:
            top2 = -np.sort(-v.reshape(G, gs), axis=1)[:, :2]
            gsc = (top2[:, 0] + top2[:, 1]).astype(F32) if gs >= 2 else top2[:, 0]
            kept = [g for g in range(G)
                    if sum(_beats(gsc[h], h, gsc[g], g) for h in range(G) if h != g) < Gk]
            assert len(kept) == Gk
            assert set((row // gs).tolist()) <= set(kept)
            allowed = np.zeros(E, dtype=bool)
            for g in kept:
                allowed[g * gs:(g + 1) * gs] = True
        else:
            allowed = np.ones(E, dtype=bool)
        assert allowed[row].all()
        # no allowed expert left out ranks above a chosen one
        out = np.flatnonzero(allowed & ~np.isin(np.arange(E), row))
        for c in row:
            for u in out:
                assert _beats(v[c], c, v[u], u), (t, c, u)
        # slots hold the chosen experts in rank order
        for a in range(k - 1):
            assert _beats(v[row[a]], row[a], v[row[a + 1]], row[a + 1])
        # gates, from the unbiased scores
        g64 = w[t].astype(np.float64)
        assert np.all(g64 >= 0)
        gamma = float(cfg.routed_scale)
        if cfg.score_fn == "sigmoid":
            s = score[t, row].astype(np.float64)
            ref = gamma * s / s.sum() if cfg.renormalize else gamma * s
        else:
            l64 = logits[t].astype(np.float64)
            if cfg.renormalize:
                e = np.exp(l64[row] - l64[row].max())
                ref = gamma * e / e.sum()
            else:
                e = np.exp(l64 - l64.max())
                ref = gamma * e[row] / e.sum()
        np.testing.assert_allclose(g64, ref, rtol=2e-5, atol=1e-30)
        if cfg.renormalize:
            assert abs(g64.sum() - gamma) <= 2e-5 * gamma


@st.composite
def dispatch_case(draw):
    E = draw(st.sampled_from([4, 8, 16, 32]))
    k = draw(st.integers(1, min(8, E)))
    T = draw(st.integers(0, 60))
    b = draw(st.integers(0, E - 1))
    e = draw(st.integers(b + 1, E))
    cf = draw(st.sampled_from([0.0, 0.25, 0.5, 1.0, 1.25]))
    skew = draw(st.sampled_from([0.0, 1.1, 2.0]))
    rng = np.random.default_rng(draw(st.integers(0, 2 ** 31 - 1)))
    p = np.arange(1, E + 1, dtype=np.float64) ** -skew
    p /= p.sum()
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        ids[t] = rng.choice(E, size=k, replace=False, p=p)
    cfg = O.Config(hidden=8, n_experts=E, top_k=k, inter=8, expert_begin=b, expert_end=e, capacity_factor=cf)
    return cfg, ids


@settings(**SETTINGS)
@given(dispatch_case())
def test_dispatch_properties(case):
    cfg, ids = case
    T, k = ids.shape
    P, b, El = T * k, cfg.expert_begin, cfg.n_local
    d = O.dispatch(cfg, ids)
    flat = ids.reshape(-1)
    # capacity: ceil(cf * T * k / E) with the global E, none when cf <= 0
    C = int(np.ceil(np.float64(F32(cfg.capacity_factor)) * T * k / cfg.n_experts)) if cfg.capacity_factor > 0 else P
    raw = np.array([np.count_nonzero(flat == b + x) for x in range(El)], dtype=np.int64)
    assert np.array_equal(d["raw_counts"], raw)
    counts = np.minimum(raw, C)
    assert np.array_equal(d["counts"], counts)
    off = np.concatenate([[0], np.cumsum(counts)])
    assert np.array_equal(d["offsets"], off)
    R = int(off[-1])
    perm, inv = np.asarray(d["perm"]), np.asarray(d["inv"])
    assert perm.shape == (R,) and inv.shape == (P,)
    # bijection between rows and kept pairs
    assert np.array_equal(np.sort(perm), np.sort(np.flatnonzero(inv >= 0)))
    for r in range(R):
        assert inv[perm[r]] == r
    for x in range(El):
        seg = perm[off[x]:off[x + 1]]
        assert np.all(flat[seg] == b + x)                    # rows of expert x hold its pairs
        assert np.all(np.diff(seg) > 0)                      # in pair order
        assert np.array_equal(seg, np.flatnonzero(flat == b + x)[:C])   # its first C pairs
    # pairs of experts outside the share, and dropped ones, have no row
    assert np.all(inv[(flat < b) | (flat >= b + El)] == -1)
    assert np.count_nonzero(inv >= 0) == R
