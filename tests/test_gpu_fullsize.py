"""Parity at the full workload sizes, in the launch configuration the
benchmark times (moe_forward, bf16 output, prepacked gate/up weights for the
bf16 layers), and at 32 times the EP8 decode batch.

At these sizes the oracle cannot run the whole layer in seconds, so:
  * routing ids and gates of EVERY token are compared bit for bit with the
    oracle's top-k on the same logits, and dispatch (counts, offsets,
    permutation, inverse permutation, capacity drops) bit for bit too;
  * the router logits and the layer output are compared on a sample of
    tokens (first, last, random ones and, with a capacity limit, tokens that
    lost an expert), the oracle computing each sampled token alone from the
    whole batch's routing.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_10_amd as moe
from oracle import moe_oracle as O
from synth import make_inputs, workload

from gpu_helpers import TOL, check_rows, host, say

pytestmark = pytest.mark.gpu

FULL = ["ep8_decode_bf16", "full_decode_bf16", "full_prefill_bf16", "fp8_skew", "full_decode_mxfp4",
        # the largest batch tested: 65536 tokens at the EP8 share (524288
        # (token, slot) pairs; about 2048 rows per local expert, so the routed
        # experts take the 256 x 256 tiles and the shared expert runs after them)
        ("ep8_decode_bf16", 65536)]


@pytest.mark.parametrize("name", FULL, ids=lambda n: n if isinstance(n, str) else f"{n[0]}_T{n[1]}")
def test_full_size_forward(name):
    w = workload(name) if isinstance(name, str) else workload(name[0], T=name[1])
    name = name if isinstance(name, str) else f"{name[0]}_T{name[1]}"
    T, k, E, H = w["T"], w["top_k"], w["n_experts"], w["hidden"]
    say("full-size case", name, "T", T)
    cfg = moe.config_from_workload(w, out_dtype="bf16")
    ocfg = O.Config.from_workload(w)
    inp = make_inputs(w, device="cuda")
    Wt = moe.make_weights(cfg, inp["w13"], inp["w2"], inp["shared_w13"], inp["shared_w2"], inp.get("w13_scale"),
                          inp.get("w2_scale"), inp.get("shared_w13_scale"), inp.get("shared_w2_scale"))
    if w["dtype"] == "bf16":
        # as bench.py runs it: the gate/up GEMMs' 256 x 256 tiles read the prepacked copy
        packed = moe.moe_prepack_weights(cfg, Wt)
        Wt = moe.make_weights(cfg, inp["w13"], inp["w2"], inp["shared_w13"], inp["shared_w2"], packed=packed)
    ws = moe.workspace(cfg, T)
    y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    say("  moe_forward")
    moe.moe_forward(cfg, inp["x"], inp["w_router"], inp["router_bias"], inp["score_bias"], Wt, y, ws,
                    logits_out=logits, topk_ids_out=ids)
    torch.cuda.synchronize()
    say("  moe_route / moe_dispatch on the same logits")
    gates = torch.empty(T, k, dtype=torch.float32, device="cuda")
    ids2 = torch.empty_like(ids)
    moe.moe_route(cfg, logits, inp["score_bias"], ids2, gates)
    El = cfg.n_local
    d = dict(raw_counts=torch.empty(El, dtype=torch.int32, device="cuda"),
             counts=torch.empty(El, dtype=torch.int32, device="cuda"),
             offsets=torch.empty(El + 1, dtype=torch.int32, device="cuda"),
             perm=torch.empty(T * k, dtype=torch.int32, device="cuda"),
             inv=torch.empty(T * k, dtype=torch.int32, device="cuda"))
    moe.moe_dispatch(cfg, ids, d["raw_counts"], d["counts"], d["offsets"], d["perm"], d["inv"], ws)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2)

    # routing and dispatch of every token, bit for bit
    l_h = host(logits)
    ref_ids, ref_w = O.route(ocfg, l_h, host(inp["score_bias"]))
    assert np.array_equal(host(ids), ref_ids)
    assert np.array_equal(host(gates).view(np.int32), ref_w.view(np.int32))
    ref_d = O.dispatch(ocfg, ref_ids)
    for key in ("raw_counts", "counts", "offsets", "inv"):
        assert np.array_equal(host(d[key]), ref_d[key]), key
    R = int(ref_d["offsets"][-1])
    assert np.array_equal(host(d["perm"])[:R], ref_d["perm"])
    dropped = int((ref_d["raw_counts"] - ref_d["counts"]).sum())
    say("  routing/dispatch bit-exact; rows", R, "dropped", dropped)

    # sampled tokens: logits and layer output
    rng = np.random.default_rng(11)
    tok = {0, T - 1, *rng.choice(T, 5, replace=False).tolist()}
    inv = ref_d["inv"].reshape(T, k)
    lost = np.nonzero((inv < 0).any(axis=1) & ((ref_ids >= w["expert_begin"]) & (ref_ids < w["expert_end"])).all(axis=1))[0]
    if len(lost):
        tok.add(int(lost[0]))
    tok = sorted(tok)
    x_s = host(inp["x"][tok])
    want_l = O.router_logits(x_s, host(inp["w_router"]), host(inp["router_bias"]))
    assert O.rel_max_err(l_h[tok], want_l) < 1e-5

    def get_expert(le):
        return (host(inp["w13"][le]), host(inp["w2"][le]),
                host(inp["w13_scale"][le]) if inp.get("w13_scale") is not None else None,
                host(inp["w2_scale"][le]) if inp.get("w2_scale") is not None else None)

    sh = None
    if w["shared_inter"]:
        sh = (host(inp["shared_w13"]), host(inp["shared_w2"]), host(inp.get("shared_w13_scale")),
              host(inp.get("shared_w2_scale")))
    say("  oracle on tokens", tok)
    want_y = O.forward_tokens(ocfg, tok, x_s, ref_ids, ref_w, ref_d["inv"], get_expert, sh)
    err = O.rel_max_err(host(y)[tok], want_y)
    say("  max|dy|/rms on the sample =", err)
    assert err < TOL[w["dtype"]]

    # whole expert groups: the routed rows of several experts, every row,
    # against the oracle's expert FFN on the same gathered tokens
    say("  moe_expert_ffn at full size")
    rd = torch.bfloat16 if w["dtype"] != "f32" else torch.float32
    rows = torch.empty(T * k, H, dtype=rd, device="cuda")
    shared = torch.empty(T, H, dtype=torch.float32, device="cuda") if w["shared_inter"] else None
    moe.moe_expert_ffn(cfg, inp["x"], d["perm"], d["offsets"], Wt, rows, shared, ws)
    torch.cuda.synchronize()
    offs = ref_d["offsets"]
    for le in _groups_to_check(ref_d):
        a, b = int(offs[le]), int(offs[le + 1])
        idx = _rows_to_check(b - a)
        say(f"  expert {le}: {b - a} rows (raw {int(ref_d['raw_counts'][le])}), checking {len(idx)}")
        toks = ref_d["perm"][a:b][idx] // k
        w13, w2, s13, s2 = get_expert(le)
        want = O.swiglu_expert(ocfg, host(inp["x"][torch.from_numpy(toks).cuda()]), w13, w2, w["inter"], s13, s2)
        got = host(rows[a:b])[idx].astype(np.float64)
        check_rows(got, want, w["dtype"])


def _groups_to_check(d):
    """The largest group; the largest whose row count is not a multiple of 32
    (a ragged last row block); a capacity-capped group, if any; the smallest
    non-empty group."""
    counts, raw = d["counts"], d["raw_counts"]
    pick = [int(np.argmax(counts))]
    ragged = np.nonzero(counts % 32)[0]
    if len(ragged):
        pick.append(int(ragged[np.argmax(counts[ragged])]))
    capped = np.nonzero(raw > counts)[0]
    if len(capped):
        pick.append(int(capped[0]))
    nz = np.nonzero(counts)[0]
    pick.append(int(nz[np.argmin(counts[nz])]))
    return list(dict.fromkeys(pick))


def _rows_to_check(n):
    """Every row of a group up to 1024 rows; beyond that the first 256 and the
    last 256 (first and last row tiles)."""
    if n <= 1024:
        return np.arange(n)
    return np.concatenate([np.arange(256), np.arange(n - 256, n)])
