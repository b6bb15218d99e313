"""Seeded random sweeps of the integer stages on the GPU against the oracle,
bit for bit: 40 router configurations (expert counts 8..512, group structures,
k up to 16, both score functions, renormalisation, scaling factor, bias, with
adversarial logits) and 30 dispatch configurations (local shares, capacity,
skew, batches on both sides of the dispatch block-length switch at 16384
pairs), bit for bit; and 16 random small layers (bf16 and fp32: expert
counts, groups, k, hidden and intermediate sizes, local shares, capacity,
score functions, biases, T up to 700, with and without a shared expert), every
stage against the oracle to the tolerances of the fixed layer cases. Every
drawn configuration satisfies the library's validation rules.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_10_amd as moe
from oracle import moe_oracle as O

from gpu_helpers import host, say

pytestmark = pytest.mark.gpu
F32 = np.float32


def _router_cfgs(n, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.choice([8, 16, 32, 48, 64, 96, 128, 160, 256, 384, 512]))
        groups = [g for g in (1, 2, 4, 8, 16, 32, 64) if E % g == 0 and (g == 1 or E // g >= 2)]
        G = int(rng.choice(groups))
        Gk = int(rng.integers(1, G + 1))
        k = int(rng.integers(1, min(16, Gk * (E // G)) + 1))
        fn = str(rng.choice(["softmax", "sigmoid"]))
        out.append(dict(E=E, G=G, Gk=Gk, k=k, fn=fn, renorm=bool(rng.integers(0, 2)),
                        gamma=float(rng.choice([1.0, 2.5])), bias=fn == "sigmoid" and bool(rng.integers(0, 2)),
                        T=int(rng.integers(1, 400)), seed=int(rng.integers(0, 2 ** 31))))
    return out


def _logits(T, E, rng):
    l = rng.standard_normal((T, E)).astype(F32)
    kind = rng.integers(0, 4, size=T)
    l[kind == 1] = np.round(l[kind == 1] * 2) / 2                    # exact ties
    l[kind == 2] = l[kind == 2] * 40                                 # saturated
    l[kind == 3] = np.where(rng.random((int((kind == 3).sum()), E)) < 0.5, F32(0.0), F32(-0.0))   # +0 / -0
    return l.astype(F32)


@pytest.mark.parametrize("i,c", list(enumerate(_router_cfgs(40))), ids=lambda v: str(v) if isinstance(v, int) else "")
def test_route_random_configs_bit_exact(i, c):
    rng = np.random.default_rng(c["seed"])
    T, E = c["T"], c["E"]
    logits = _logits(T, E, rng)
    sb = (rng.standard_normal(E) * 0.1).astype(F32) if c["bias"] else None
    say("route sweep", i, c)
    cfg = moe.make_config(512, E, c["k"], 128, n_group=c["G"], topk_group=c["Gk"], score_fn=c["fn"],
                          renormalize=c["renorm"], routed_scale=c["gamma"], dtype="bf16")
    ids = torch.empty(T, c["k"], dtype=torch.int32, device="cuda")
    w = torch.empty(T, c["k"], dtype=torch.float32, device="cuda")
    moe.moe_route(cfg, torch.from_numpy(logits).cuda(), None if sb is None else torch.from_numpy(sb).cuda(), ids, w)
    ocfg = O.Config(hidden=512, n_experts=E, top_k=c["k"], inter=128, n_group=c["G"], topk_group=c["Gk"],
                    score_fn=c["fn"], renormalize=c["renorm"], routed_scale=c["gamma"])
    oid, ow = O.route(ocfg, logits, sb)
    gid, gw = host(ids), host(w)
    assert np.array_equal(gid, oid), np.argwhere(gid != oid)[:5]
    assert np.array_equal(gw.view(np.int32), ow.view(np.int32)), np.argwhere(gw != ow)[:5]


def _dispatch_cfgs(n, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(rng.choice([8, 16, 64, 128, 256, 512]))
        k = int(rng.integers(1, min(16, E) + 1))
        T = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 3000)),
                            int(rng.integers(16384 // k - 2, 16384 // k + 3)), int(rng.integers(3000, 20000 // k + 3001))]))
        b = int(rng.integers(0, E))
        e = int(rng.integers(b + 1, E + 1))
        out.append(dict(T=max(T, 1), E=E, k=k, b=b, e=e, cf=float(rng.choice([0.0, 0.5, 1.0, 1.25, 2.0])),
                        skew=float(rng.choice([0.0, 1.1, 2.0])), seed=int(rng.integers(0, 2 ** 31))))
    return out


def _ids(T, E, k, rng, skew):
    p = np.arange(1, E + 1, dtype=np.float64) ** -skew
    p /= p.sum()
    g = rng.random((T, E)) ** (1.0 / p)          # weighted sampling without replacement
    return np.argsort(-g, axis=1)[:, :k].astype(np.int32)


@pytest.mark.parametrize("i,c", list(enumerate(_dispatch_cfgs(30))), ids=lambda v: str(v) if isinstance(v, int) else "")
def test_dispatch_random_configs_bit_exact(i, c):
    rng = np.random.default_rng(c["seed"])
    T, E, k, b, e = c["T"], c["E"], c["k"], c["b"], c["e"]
    ids = _ids(T, E, k, rng, c["skew"])
    say("dispatch sweep", i, c)
    cfg = moe.make_config(512, E, k, 128, expert_begin=b, expert_end=e, dtype="bf16", capacity_factor=c["cf"])
    ocfg = O.Config(hidden=512, n_experts=E, top_k=k, inter=128, expert_begin=b, expert_end=e,
                    capacity_factor=c["cf"])
    ref = O.dispatch(ocfg, ids)
    El = e - b
    ws = moe.workspace(cfg, T)
    o = dict(raw_counts=torch.empty(El, dtype=torch.int32, device="cuda"),
             counts=torch.empty(El, dtype=torch.int32, device="cuda"),
             offsets=torch.empty(El + 1, dtype=torch.int32, device="cuda"),
             perm=torch.full((T * k,), -7, dtype=torch.int32, device="cuda"),
             inv=torch.empty(T * k, dtype=torch.int32, device="cuda"))
    moe.moe_dispatch(cfg, torch.from_numpy(ids).cuda(), o["raw_counts"], o["counts"], o["offsets"], o["perm"],
                     o["inv"], ws)
    got = {key: host(v) for key, v in o.items()}
    R = int(ref["offsets"][-1])
    for key in ("raw_counts", "counts", "offsets", "inv"):
        assert np.array_equal(got[key], ref[key]), key
    assert np.array_equal(got["perm"][:R], ref["perm"])
    assert np.all(got["perm"][R:] == -7)


def _layer_cfgs(n, seed=31):
    """Random small layers, bf16 and fp32 (the e4m3 / FP4 paths have their
    own cases at the model's intermediate sizes, where requantisation flips
    stay rare)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        dtype = str(rng.choice(["bf16", "bf16", "bf16", "f32"]))
        E = int(rng.choice([8, 16, 32, 64, 128]))
        groups = [g for g in (1, 2, 4, 8) if E % g == 0 and (g == 1 or E // g >= 2)]
        G = int(rng.choice(groups))
        Gk = int(rng.integers(1, G + 1))
        k = int(rng.integers(1, min(8, Gk * (E // G)) + 1))
        H = int(rng.choice([128, 256, 512] if dtype == "f32" else [256, 512, 1024]))
        I = int(rng.choice([128, 256, 384, 640]))
        b = int(rng.integers(0, E // 2))
        e = int(rng.integers(b + 1, E + 1))
        fn = str(rng.choice(["softmax", "sigmoid"]))
        T = int(rng.integers(1, 300 if dtype == "f32" else 700))
        out.append(dict(name=f"sweep{len(out)}", T=T, hidden=H, n_experts=E, expert_begin=b, expert_end=e, top_k=k,
                        n_group=G, topk_group=Gk, score_fn=fn, renormalize=bool(rng.integers(0, 2)),
                        routed_scale=float(rng.choice([1.0, 2.5])), inter=I,
                        shared_inter=int(rng.choice([0, 128, 256, 384])), dtype=dtype,
                        capacity_factor=float(rng.choice([0.0, 0.0, 1.0, 1.5])),
                        score_bias=("normal0.1" if fn == "sigmoid" and rng.integers(0, 2) else "none"),
                        router_bias=str(rng.choice(["none", "zipf1.1"]))))
    return out


@pytest.mark.parametrize("w", _layer_cfgs(16), ids=lambda w: w["name"])
def test_layer_random_configs(w):
    from test_gpu_parity import check_layer
    check_layer(w, w["name"])
