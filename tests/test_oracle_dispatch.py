"""Pins of the oracle's dispatch (per-expert counts, offsets, permutation) and
capacity rule: invariants, numpy's stable argsort as a brute-force reference,
and the closed-form capacity of the skewed fp8 workload (1.25 * 8192 * 8 / 256)."""
import numpy as np
import pytest

from oracle import moe_oracle as O


def _cfg(**kw):
    base = dict(hidden=8, n_experts=16, top_k=4, inter=8)
    base.update(kw)
    return O.Config(**base)


def _ids(T, E, k, seed, skew=0.0):
    rng = np.random.default_rng(seed)
    p = np.exp(-skew * np.log(np.arange(1, E + 1)))
    p /= p.sum()
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        out[t] = rng.choice(E, size=k, replace=False, p=p)
    return out


def _check(cfg, ids, d):
    T, k = ids.shape
    P = T * k
    El, b = cfg.n_local, cfg.expert_begin
    C = O.capacity(cfg, T)
    flat = ids.reshape(-1)
    local = (flat >= b) & (flat < b + El)
    raw_ref = np.bincount(flat[local] - b, minlength=El)
    assert np.array_equal(d["raw_counts"], raw_ref)
    cnt_ref = raw_ref if C is None else np.minimum(raw_ref, C)
    assert np.array_equal(d["counts"], cnt_ref)
    assert d["offsets"][0] == 0 and np.array_equal(np.diff(d["offsets"]), cnt_ref)
    R = d["offsets"][-1]
    kept = d["inv"] >= 0
    dropped = local & ~kept
    assert kept.sum() == R and R + dropped.sum() + (~local).sum() == P
    # perm o inv is the identity on kept pairs; inv o perm on rows
    assert np.array_equal(d["perm"][d["inv"][kept]], np.flatnonzero(kept))
    assert np.array_equal(d["inv"][d["perm"]], np.arange(R))
    # brute force: stable argsort of the kept pairs by expert
    kp = np.flatnonzero(kept)
    assert np.array_equal(d["perm"], kp[np.argsort(flat[kp], kind="stable")])
    # capacity keeps the first C pairs of each expert, in pair order
    if C is not None:
        for e in range(El):
            pe = np.flatnonzero(flat == b + e)
            assert np.array_equal(np.sort(d["perm"][d["offsets"][e]:d["offsets"][e + 1]]), pe[:C])


@pytest.mark.parametrize("T,E,k,b,e,cf,skew", [
    (64, 16, 4, 0, 16, 0.0, 0.0),
    (200, 16, 4, 4, 12, 0.0, 0.0),     # local share
    (300, 16, 2, 0, 16, 1.25, 1.1),    # capacity with skew
    (100, 16, 4, 8, 16, 1.0, 1.5),     # capacity + share
    (1, 16, 4, 0, 16, 0.0, 0.0),
])
def test_dispatch_invariants_and_argsort(T, E, k, b, e, cf, skew):
    cfg = _cfg(n_experts=E, top_k=k, expert_begin=b, expert_end=e, capacity_factor=cf)
    ids = _ids(T, E, k, seed=T + E + k, skew=skew)
    _check(cfg, ids, O.dispatch(cfg, ids))


def test_dispatch_empty_batch():
    cfg = _cfg()
    d = O.dispatch(cfg, np.zeros((0, 4), dtype=np.int32))
    assert d["perm"].size == 0 and d["inv"].size == 0 and np.all(d["offsets"] == 0)


def test_capacity_closed_form_fp8_workload():
    cfg = _cfg(n_experts=256, top_k=8, capacity_factor=1.25)
    assert O.capacity(cfg, 8192) == 320
    assert O.capacity(_cfg(capacity_factor=0.0), 8192) is None
    # ceil: 1.25 * 10 * 4 / 16 = 3.125 -> 4
    assert O.capacity(_cfg(capacity_factor=1.25), 10) == 4


def test_dispatch_capacity_drops_counted():
    cfg = _cfg(n_experts=4, top_k=1, capacity_factor=1.0)   # C = T/4
    ids = np.array([[0]] * 6 + [[1]] * 2, dtype=np.int32)
    d = O.dispatch(cfg, ids)
    assert O.capacity(cfg, 8) == 2
    assert d["raw_counts"].tolist() == [6, 2, 0, 0] and d["counts"].tolist() == [2, 2, 0, 0]
    assert d["inv"].tolist() == [0, 1, -1, -1, -1, -1, 2, 3]
    assert d["perm"].tolist() == [0, 1, 6, 7]
