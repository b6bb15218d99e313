"""The prepacked gate/up and down weight layout and the grouped GEMMs that
read it.

moe_prepack_weights is pure data movement: its output is compared byte for
byte with the layout the header documents, computed here with numpy indexing.
Layers whose expert GEMMs take the 256 x 256 compute-bound tiles are run with
and without the packed copy: the two kernels accumulate K in the same order
with the same MFMA instruction, so expert rows, shared output and y must be
equal bit for bit; and the packed run is held to the oracle stage by stage.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_10_amd as moe
from synth import make_inputs, workload

from gpu_helpers import Run, host, say
from test_gpu_parity import _small, check_layer

pytestmark = pytest.mark.gpu


def _expected_packed(w, n_rows, K, inter, down=False):
    """Documented layout: panel p, K step s, half h, lane l, element e holds
    W[n][k] with n = gate row p*32 + l%32 (h = 0) or up row inter + p*32 +
    l%32 (h = 1) of a gate/up weight, row p*64 + 32 h + l%32 of a down
    weight, and k = 16 s + 8 (l // 32) + e."""
    W = w.reshape(n_rows, K)
    n_panels = n_rows // 64 if down else inter // 32
    p = np.arange(n_panels)[:, None, None, None, None]
    s = np.arange(K // 16)[None, :, None, None, None]
    h = np.arange(2)[None, None, :, None, None]
    l = np.arange(64)[None, None, None, :, None]
    e = np.arange(8)[None, None, None, None, :]
    n = (p * 64 + h * 32 + l % 32) if down else (np.where(h == 1, inter, 0) + p * 32 + l % 32)
    k = s * 16 + (l // 32) * 8 + e
    return W[n, k].reshape(-1)


@pytest.mark.parametrize("H,I,Is,El", [(512, 256, 256, 3), (640, 384, 128, 2), (7168, 2048, 2048, 1)])
def test_prepack_layout_byte_exact(H, I, Is, El):
    say("prepack layout", H, I, Is, El)
    cfg = moe.make_config(H, 8, 2, I, expert_end=El, shared_inter=Is, dtype="bf16")
    g = torch.Generator(device="cuda").manual_seed(H + I)
    mk = lambda *shape: torch.randn(*shape, generator=g, device="cuda").to(torch.bfloat16)
    w13, w2, s13, s2 = mk(El, 2 * I, H), mk(El, H, I), mk(2 * Is, H), mk(H, Is)
    W = moe.make_weights(cfg, w13, w2, s13, s2)
    nbytes = moe.packed_weights_bytes(cfg)
    packed = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
    moe.moe_prepack_weights(cfg, W, packed)
    torch.cuda.synchronize()
    got = packed.cpu().view(torch.int16).numpy()
    bits = lambda t: t.cpu().view(torch.int16).numpy()
    al = lambda b: (b + 255) // 256 * 256
    off = 0
    for e in range(El):
        want = _expected_packed(bits(w13[e]), 2 * I, H, I)
        assert np.array_equal(got[off // 2 + e * 2 * I * H: off // 2 + (e + 1) * 2 * I * H], want), ("w13", e)
    off += al(2 * El * 2 * I * H)
    assert np.array_equal(got[off // 2: off // 2 + 2 * Is * H], _expected_packed(bits(s13), 2 * Is, H, Is))
    off += al(2 * 2 * Is * H)
    for e in range(El):
        want = _expected_packed(bits(w2[e]), H, I, None, down=True)
        assert np.array_equal(got[off // 2 + e * H * I: off // 2 + (e + 1) * H * I], want), ("w2", e)
    assert off + al(2 * El * H * I) == nbytes


# layers whose expert GEMMs take the 256 x 256 tiles
PACKED_CASES = {
    # routed experts on 256 x 256 tiles (about 256 rows per expert), shared expert too
    "big_tiles": lambda: _small(T=2048, n_experts=32, expert_end=32, top_k=4, n_group=4, topk_group=2,
                                inter=2048, shared_inter=2048, score_bias="zero"),
    # K stages not a multiple of four (hidden 640: 10 stages, inter 384: 6),
    # an output tile with two of its four panels past the last one, ragged tiles
    "ragged_k_and_panels": lambda: _small(T=11000, hidden=640, n_experts=16, expert_end=16, top_k=4, n_group=4,
                                          topk_group=2, inter=384, shared_inter=384, score_bias="zero"),
    # two K stages in both GEMMs (hidden 128, inter 128): the shortest K loop
    # (one column tile each, so 32768 tokens for enough 256-row tiles)
    "two_k_stages": lambda: _small(T=32768, hidden=128, n_experts=16, expert_end=16, top_k=4, n_group=4,
                                   topk_group=2, inter=128, shared_inter=128, score_bias="zero"),
    # capacity-capped groups of uneven size on the packed tiles, a local share
    "capacity_share": lambda: _small(T=4200, hidden=512, n_experts=16, expert_begin=2, expert_end=14, top_k=4,
                                     n_group=4, topk_group=2, inter=1024, shared_inter=512, capacity_factor=1.25,
                                     router_bias="zipf1.1", score_bias="zero"),
    # the shared expert on packed 256 x 256 tiles beside routed decode tiles
    "shared_only_big": lambda: _small(T=1100, expert_end=16, shared_inter=512),
}


@pytest.mark.parametrize("name", list(PACKED_CASES))
def test_packed_equals_unpacked_bit_for_bit(name):
    w = PACKED_CASES[name]()
    say("packed vs unpacked", name, {k: w[k] for k in ("T", "hidden", "inter", "shared_inter")})
    a = Run(w).stages()
    b = Run(w, packed=True).stages()
    for key in ("ids", "offsets", "perm"):
        assert torch.equal(a[key], b[key]), key
    R = int(a["offsets"][-1])
    assert torch.equal(a["rows"][:R], b["rows"][:R])
    if a["shared"] is not None:
        assert torch.equal(a["shared"], b["shared"])
    assert torch.equal(a["y"], b["y"])


@pytest.mark.parametrize("name", list(PACKED_CASES))
def test_packed_layer_matches_oracle(name):
    check_layer(PACKED_CASES[name](), f"packed_{name}", packed=True)


def test_packed_share_at_64_rows_per_expert_matches_oracle():
    """An expert-parallel share at about 64 rows per expert: with packed
    weights the routed GEMMs take the 256 x 256 packed tiles from 32 rows per
    expert on (tiles of 1-3 row blocks), without them the decode tiles, so
    only the oracle decides here."""
    w = _small(T=2048, hidden=256, n_experts=128, expert_end=32, top_k=4, n_group=4, topk_group=2, inter=2048,
               shared_inter=512, score_bias="zero")
    check_layer(w, "packed_share_64_rows", packed=True)
