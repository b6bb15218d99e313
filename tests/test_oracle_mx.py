"""Pins of the oracle's microscaling (MX) arithmetic: FP4 weights and MX e4m3
activations.

References, none of them the oracle's own formulas:
  * the E2M1 value table and the E8M0 scale rule of the OCP microscaling
    formats (written out as literal values);
  * a brute-force search for each block's shared exponent and each element's
    nearest e4m3 value (every finite e4m3 value enumerated from torch's
    float8 dtype, ties to the even code);
  * element-by-element Python loops for the packed layout;
  * torch's float8_e4m3fn cast and F.linear / F.silu for the expert FFN;
  * the bf16 oracle on the same dequantised weights, within the error bound
    of the activation quantisation.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O
from synth import make_inputs, workload

# OCP MX E2M1: codes 0..7 positive, 8..15 the same magnitudes negated.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
              -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_decode_all_codes():
    got = O.e2m1_decode(np.arange(16))
    assert got.tolist() == E2M1_TABLE
    assert np.signbit(got[8])                      # code 8 is -0


def test_e8m0_decode():
    got = O.e8m0_decode(np.array([0, 1, 120, 126, 127, 128, 200, 254, 255]))
    assert got[:8].tolist() == [2.0 ** -127, 2.0 ** -126, 2.0 ** -7, 0.5, 1.0, 2.0, 2.0 ** 73, 2.0 ** 127]
    assert math.isnan(got[8])


def test_fp4_weight_layout_element_by_element():
    rng = np.random.default_rng(3)
    n, k = 5, 96
    packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = rng.integers(120, 135, size=(n, k // 32), dtype=np.uint8)
    got = O.dequant_mx_weight(packed, scales)
    for r in range(n):
        for c in range(k):
            byte = int(packed[r, c // 2])
            code = (byte >> 4) if c % 2 else (byte & 15)
            want = E2M1_TABLE[code] * 2.0 ** (int(scales[r, c // 32]) - 127)
            assert got[r, c] == want, (r, c)


def test_fp4_weight_layout_one_hot():
    packed = np.zeros((4, 64), dtype=np.uint8)
    scales = np.full((4, 4), 127, dtype=np.uint8)
    packed[3, 5] = 0x02                                 # low nibble: element 10 = 1.0
    packed[1, 20] = 0xF0                                # high nibble: element 41 = -6.0
    scales[1, 1] = 129                                  # elements 32..63 of row 1 times 4
    w = O.dequant_mx_weight(packed, scales)
    nz = np.argwhere(w != 0)
    assert nz.tolist() == [[1, 41], [3, 10]]
    assert w[3, 10] == 1.0 and w[1, 41] == -24.0


def _e4m3_grid():
    """Every finite non-negative e4m3fn value with its code (torch's dtype)."""
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)           # 0x7F is NaN
    vals = codes.view(torch.float8_e4m3fn).double().numpy()
    return vals, codes.numpy()


def _brute_mx(v):
    """Shared exponent by search, then the nearest e4m3 value by search."""
    vals, codes = _e4m3_grid()
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    rows, cols = v.shape
    q = np.zeros_like(v)
    sc = np.zeros((rows, cols // 32), dtype=np.int64)
    for r in range(rows):
        for b in range(cols // 32):
            blk = v[r, 32 * b:32 * b + 32]
            a = np.max(np.abs(blk))
            if a == 0:
                x = -127
            else:
                # the X that brings the block maximum into [256, 512) = [2**8, 2**9)
                x = next(x for x in range(-300, 300) if 256.0 <= a * 2.0 ** -x < 512.0)
                x = min(max(x, -127), 127)
            sc[r, b] = x + 127
            for i, e in enumerate(blk):
                t = min(abs(e) * 2.0 ** -x, 448.0)
                d = np.abs(vals - t)
                best = np.flatnonzero(d == d.min())
                if len(best) > 1:                               # a tie: the even code
                    best = [c for c in best if codes[c] % 2 == 0]
                m = vals[best[0]]
                q[r, 32 * b + i] = -m if e < 0 else m
    return q, sc


def test_quantize_mx_rows_matches_brute_force():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((6, 128)).astype(np.float32)
    v[1] *= 1e-3
    v[2, :32] = 0.0                                     # zero block
    v[3, 32:64] = 2.0 ** rng.integers(-3, 4, 32)         # powers of two: exact
    v[3, 64:96] *= 2.0 ** -40                            # tiny but normal
    v[4, :32] = np.linspace(-1.99, 1.99, 32)             # amax just below a power of two: saturates
    v[5, :32] = 0.0
    v[5, 0] = 1.0625                                     # 272 after scaling: midway 256..288, to 256 (even)
    v[5, 1] = -1.1875                                    # 304: midway 288..320, to 320 (even)
    q, sc = O.quantize_mx_rows(v)
    bq, bsc = _brute_mx(v)
    assert np.array_equal(sc.astype(np.int64), bsc)
    assert np.array_equal(q, bq)
    deq = O.dequant_mx_rows(q, sc)
    assert deq[5, 0] == 1.0 and deq[5, 1] == -1.25
    assert np.array_equal(deq[3, 32:64], v[3, 32:64].astype(np.float64))
    assert np.all(deq[2, :32] == 0)


def test_quantize_mx_rows_subnormal_range_and_bounds():
    # blocks whose maximum sits far below 2**-119 clamp the exponent at -127
    v = np.zeros((2, 64), dtype=np.float32)
    v[0, :32] = np.float32(2.0 ** -130) * np.arange(1, 33, dtype=np.float32)
    v[1, :32] = np.float32(2.0 ** 126) * np.linspace(-1.5, 1.5, 32, dtype=np.float32)
    q, sc = O.quantize_mx_rows(v)
    bq, bsc = _brute_mx(v)
    assert sc[0, 0] == 0 and np.array_equal(sc.astype(np.int64), bsc) and np.array_equal(q, bq)
    # every dequantised element is within the e4m3 half-step of its value or
    # saturated at 448 * 2**X (blocks of normal data)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    q, sc = O.quantize_mx_rows(x)
    deq = O.dequant_mx_rows(q, sc)
    s = np.repeat(O.e8m0_decode(sc), 32, axis=1)
    assert np.all(np.abs(q) <= 448)
    inside = np.abs(x) <= 448 * s
    assert np.all(np.abs(deq - x)[inside] <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s)[inside])
    assert np.all(np.abs(deq)[~inside] == (448 * s)[~inside])


def _tiny(**kw):
    w = dict(T=40, hidden=256, n_experts=8, expert_begin=0, expert_end=8, top_k=2,
             n_group=1, topk_group=1, score_fn="softmax", renormalize=True,
             routed_scale=1.0, inter=128, shared_inter=0, dtype="mxfp4",
             capacity_factor=0.0, score_bias="none", router_bias="none")
    w.update(kw)
    return w


def test_mx_expert_matches_torch_casts():
    """The expert FFN with MX activations, rebuilt from torch's e4m3 cast."""
    w = _tiny()
    inp = make_inputs(w)
    cfg = O.Config.from_workload(w)
    e = 3
    x = inp["x"].float()
    got = O.swiglu_expert(cfg, x.numpy(), inp["w13"][e].numpy(), inp["w2"][e].numpy(), 128,
                          inp["w13_scale"][e].numpy(), inp["w2_scale"][e].numpy())

    def deq_w(p, s):
        lo, hi = (p & 15).long(), (p >> 4).long()
        codes = torch.stack([lo, hi], -1).reshape(p.shape[0], -1)
        vals = torch.tensor(E2M1_TABLE, dtype=torch.float64)[codes]
        return vals * torch.pow(2.0, s.double() - 127).repeat_interleave(32, 1)

    def quant_act(v):           # float32 [n, K] -> dequantised float64
        b = v.reshape(v.shape[0], -1, 32)
        a = b.abs().amax(-1, keepdim=True)
        _, ex = torch.frexp(a)
        X = torch.where(a > 0, ex - 9, torch.full_like(ex, -127)).clamp(-127, 127)
        q = (b * torch.pow(2.0, -X.float())).clamp(-448, 448).to(torch.float8_e4m3fn).double()
        return (q * torch.pow(2.0, X.double())).reshape(v.shape)

    W13 = deq_w(inp["w13"][e], inp["w13_scale"][e])
    W2 = deq_w(inp["w2"][e], inp["w2_scale"][e])
    xa = quant_act(x)
    h = F.silu(F.linear(xa, W13[:128])) * F.linear(xa, W13[128:])
    ha = quant_act(h.float())
    ref = F.linear(ha, W2).to(torch.bfloat16).double().numpy()
    # h is float32 here and float64 (rounded to float32) in the oracle: a rare
    # element can land on the other side of an e4m3 rounding boundary
    err = np.abs(got - ref) / np.sqrt(np.mean(ref ** 2))
    assert np.mean(err < 1e-2) > 0.99 and err.max() < 0.1


def test_mx_layer_close_to_unquantised_layer():
    """Quantising x and h to MX e4m3 moves y by about the e4m3 step (2**-4
    relative) and no more: a dropped term, a wrong block axis or a transposed
    operand would move it by O(1)."""
    w = _tiny(shared_inter=128, score_fn="sigmoid", n_group=4, topk_group=2, top_k=3)
    inp = make_inputs(w)
    cfg = O.Config.from_workload(w)
    x = inp["x"].float().numpy()
    wr = inp["w_router"].float().numpy()
    W13 = np.stack([O.dequant_mx_weight(inp["w13"][e].numpy(), inp["w13_scale"][e].numpy()) for e in range(8)])
    W2 = np.stack([O.dequant_mx_weight(inp["w2"][e].numpy(), inp["w2_scale"][e].numpy()) for e in range(8)])
    S13 = O.dequant_mx_weight(inp["shared_w13"].numpy(), inp["shared_w13_scale"].numpy())
    S2 = O.dequant_mx_weight(inp["shared_w2"].numpy(), inp["shared_w2_scale"].numpy())
    scales = dict(w13_scale=inp["w13_scale"].numpy(), w2_scale=inp["w2_scale"].numpy(),
                  shared_w13_scale=inp["shared_w13_scale"].numpy(), shared_w2_scale=inp["shared_w2_scale"].numpy())
    got = O.forward(cfg, x, wr, inp["w13"].numpy(), inp["w2"].numpy(), shared_w13=inp["shared_w13"].numpy(),
                    shared_w2=inp["shared_w2"].numpy(), scales=scales)
    cfg64 = O.Config.from_workload(dict(w, dtype="f32"))
    ref = O.forward(cfg64, x, wr, W13, W2, shared_w13=S13, shared_w2=S2, logits=got["logits"].astype(np.float32))
    assert np.array_equal(got["ids"], ref["ids"])
    rel = np.sqrt(np.mean((got["y"] - ref["y"]) ** 2) / np.mean(ref["y"] ** 2))
    assert 0.005 < rel < 0.06
