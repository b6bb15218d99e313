"""Every instantiation of the 256 x 256 grouped-GEMM loops against the oracle.

Both 256 x 256 kernels compile their K loop once per count of 32-row blocks
that hold data (the packed gate/up kernel per tile, 1..8; the LDS-staged
kernel per wavefront row, 0..4). Routed layers reach only the counts their
routing happens to produce, so here moe_expert_ffn runs on a hand-made
dispatch whose expert groups have sizes chosen to produce every count:
single tiles of 1..8 blocks, and groups split into several row tiles
(balanced split: 257 rows -> 160 + 97, 600 -> 224 + 224 + 152, 777 ->
224 x 3 + 105). Every row of every group is held to the oracle's expert
FFN on the same gathered tokens, with packed and with canonical gate/up
weights, and the two runs must agree bit for bit (same K order).
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_10_amd as moe
from oracle import moe_oracle as O

from gpu_helpers import check_rows, host, say

pytestmark = pytest.mark.gpu

# rows per local expert: 1..8 blocks in one tile, then multi-tile groups
GROUPS = [1, 20, 33, 64, 90, 120, 150, 180, 210, 250, 256, 257, 300, 511, 600, 777]


def _blocks(rows):
    """Blocks with data of each row tile of a group (balanced split, 256-row tiles)."""
    mt = (rows + 255) // 256
    tr = min(256, ((rows + mt - 1) // mt + 31) // 32 * 32)
    return [(min(tr, rows - m * tr) + 31) // 32 for m in range(mt)]


def test_groups_cover_every_block_count():
    counts = {b for r in GROUPS for b in _blocks(r)}
    assert counts == set(range(1, 9)), counts
    # wavefront rows of the LDS-staged kernel: full tiles give 4 and 4, short
    # tiles alternate blocks, (n + 1) // 2 and n // 2
    per_wave = {c for b in counts for c in ((4, 4) if b == 8 else ((b + 1) // 2, b // 2))}
    assert per_wave == set(range(0, 5)), per_wave


@pytest.mark.parametrize("shared_inter", [0, 512])
def test_every_block_count_matches_oracle(shared_inter):
    E, k, H, I = len(GROUPS), 2, 512, 2048
    T = 4096                                   # T k / E = 512 rows expected: 256 x 256 tiles
    say("tile variants: groups", GROUPS, "shared_inter", shared_inter)
    cfg = moe.make_config(H, E, k, I, shared_inter=shared_inter, n_group=1, topk_group=1, dtype="bf16")
    ocfg = O.Config(hidden=H, n_experts=E, top_k=k, inter=I, shared_inter=shared_inter, n_group=1, topk_group=1,
                    act="bf16")
    g = torch.Generator(device="cpu").manual_seed(1234 + shared_inter)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w13 = (torch.randn(E, 2 * I, H, generator=g) / H ** 0.5).to(torch.bfloat16)
    w2 = (torch.randn(E, H, I, generator=g) / I ** 0.5).to(torch.bfloat16)
    s13 = (torch.randn(2 * shared_inter, H, generator=g) / H ** 0.5).to(torch.bfloat16) if shared_inter else None
    s2 = (torch.randn(H, shared_inter, generator=g) / shared_inter ** 0.5).to(torch.bfloat16) if shared_inter else None
    # a dispatch: each expert's rows are distinct (token, slot) pairs
    rng = np.random.default_rng(7)
    R = sum(GROUPS)
    pairs = rng.permutation(T * k)[:R].astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(GROUPS)]).astype(np.int32)
    perm = np.full(T * k, -1, dtype=np.int32)
    perm[:R] = pairs
    dev = lambda a: torch.from_numpy(a).cuda()
    xd = x.cuda()
    Wc = moe.make_weights(cfg, w13.cuda(), w2.cuda(), s13.cuda() if s13 is not None else None,
                          s2.cuda() if s2 is not None else None)
    packed = moe.moe_prepack_weights(cfg, Wc)
    Wp = moe.make_weights(cfg, w13.cuda(), w2.cuda(), s13.cuda() if s13 is not None else None,
                          s2.cuda() if s2 is not None else None, packed=packed)
    ws = moe.workspace(cfg, T)
    outs = {}
    for name, W in (("canonical", Wc), ("packed", Wp)):
        rows = torch.empty(T * k, H, dtype=torch.bfloat16, device="cuda")
        sh = torch.empty(T, H, dtype=torch.float32, device="cuda") if shared_inter else None
        moe.moe_expert_ffn(cfg, xd, dev(perm), dev(offsets), W, rows, sh, ws)
        torch.cuda.synchronize()
        outs[name] = (rows[:R].cpu(), None if sh is None else sh.cpu())
    # packed and canonical: bit for bit
    assert torch.equal(outs["packed"][0].view(torch.int16), outs["canonical"][0].view(torch.int16))
    if shared_inter:
        assert torch.equal(outs["packed"][1].view(torch.int32), outs["canonical"][1].view(torch.int32))
    # every row of every group against the oracle's expert FFN
    xh = host(x)
    got = host(outs["packed"][0]).astype(np.float64)
    for e, n in enumerate(GROUPS):
        a, b = int(offsets[e]), int(offsets[e + 1])
        toks = pairs[a:b] // k
        want = O.swiglu_expert(ocfg, xh[toks], host(w13[e]), host(w2[e]), I)
        say(f"  expert {e}: {n} rows, tiles of {_blocks(n)} blocks")
        check_rows(got[a:b], want, "bf16")
    if shared_inter:
        want = O.shared_forward(ocfg, xh, host(s13), host(s2))
        err = O.rel_max_err(host(outs["packed"][1]), want)
        say("  shared expert: max|d|/rms", err)
        assert err < 2e-2


@pytest.mark.parametrize("small_first", [True, False])
def test_work_balanced_xcd_ranges_at_their_cap(small_first):
    """The 256 x 256 launches deal their items to the 8 XCDs in ranges cut by
    estimated work, each range capped at the launch's workgroup slots per XCD.
    Half the experts with 20 rows (one-block items, cheap) and half with 1004
    (four m-tiles of full blocks): cut by work alone, the ranges over the cheap
    items would hold more items than an XCD has slots, so the cap decides
    (at this shape the ranges over the cheap items reach it exactly in the
    packed gate/up launch, 384 items, and in the down launch, 24). Every row
    starts as NaN: a lost item leaves NaN rows, a wrong one differs from the
    oracle."""
    E, k, H, I, T = 64, 8, 256, 2048, 4096
    sizes = [20] * 32 + [1004] * 32
    if not small_first:
        sizes = sizes[::-1]
    say("xcd ranges: 32 experts x 20 rows, 32 x 1004, small first:", small_first)
    cfg = moe.make_config(H, E, k, I, shared_inter=0, n_group=1, topk_group=1, dtype="bf16")
    ocfg = O.Config(hidden=H, n_experts=E, top_k=k, inter=I, shared_inter=0, n_group=1, topk_group=1, act="bf16")
    g = torch.Generator(device="cpu").manual_seed(99 + small_first)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w13 = (torch.randn(E, 2 * I, H, generator=g) / H ** 0.5).to(torch.bfloat16)
    w2 = (torch.randn(E, H, I, generator=g) / I ** 0.5).to(torch.bfloat16)
    rng = np.random.default_rng(11)
    R = sum(sizes)
    assert R <= T * k
    pairs = rng.permutation(T * k)[:R].astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    perm = np.full(T * k, -1, dtype=np.int32)
    perm[:R] = pairs
    dev = lambda a: torch.from_numpy(a).cuda()
    Wc = moe.make_weights(cfg, w13.cuda(), w2.cuda())
    packed = moe.moe_prepack_weights(cfg, Wc)
    Wp = moe.make_weights(cfg, w13.cuda(), w2.cuda(), packed=packed)
    ws = moe.workspace(cfg, T)
    outs = {}
    for name, W in (("canonical", Wc), ("packed", Wp)):
        rows = torch.full((T * k, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        moe.moe_expert_ffn(cfg, x.cuda(), dev(perm), dev(offsets), W, rows, None, ws)
        torch.cuda.synchronize()
        outs[name] = rows[:R].cpu()
    assert torch.equal(outs["packed"].view(torch.int16), outs["canonical"].view(torch.int16))
    got = host(outs["packed"]).astype(np.float64)
    assert np.isfinite(got).all()                 # every row written
    xh = host(x)
    for e, n in enumerate(sizes):
        a, b = int(offsets[e]), int(offsets[e + 1])
        want = O.swiglu_expert(ocfg, xh[pairs[a:b] // k], host(w13[e]), host(w2[e]), I)
        check_rows(got[a:b], want, "bf16")
