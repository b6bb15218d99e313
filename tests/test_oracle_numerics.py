"""Pins of the oracle's number formats and its float32 exp / sigmoid recipe.

Each check compares against something other than the oracle itself: the exact
function in fp64, torch's own bfloat16 / float8_e4m3fn casts (library
routines), closed-form code values of the OCP E4M3FN format, or invariants.
"""
import math

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

F32 = np.float32


def _ulps(a, ref64):
    a = np.asarray(a, dtype=F32)
    r = np.asarray(ref64, dtype=np.float64).astype(F32)
    return np.abs(a.view(np.int32).astype(np.int64) - r.view(np.int32).astype(np.int64))


def _sweep(hi, stride=193):
    """Non-negative float32 values <= hi, a strided walk over bit patterns."""
    bits = np.arange(0, 0x7F800000, stride, dtype=np.int64).astype(np.uint32)
    v = bits.view(F32)
    return v[v <= hi]


def test_exp_f32_within_1ulp_of_exact():
    y = -_sweep(87.0)
    e = O.exp_f32(y)
    assert _ulps(e, np.exp(y.astype(np.float64))).max() <= 1


def test_exp_f32_special_points():
    assert O.exp_f32(F32(0.0)) == F32(1.0)
    assert O.exp_f32(F32(-0.0)) == F32(1.0)
    # clamp: every argument below -87 gives e**-87 (a normal float32)
    lo = O.exp_f32(np.array([-87.0, -100.0, -1e30], dtype=F32))
    assert lo[0] == lo[1] == lo[2] and lo[0] > np.finfo(F32).tiny


def test_sigmoid_f32_within_2ulp_of_exact():
    for x in (_sweep(100.0), -_sweep(87.0)):
        s = O.sigmoid_f32(x)
        ref = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
        assert _ulps(s, ref).max() <= 2


def test_sigmoid_f32_monotone_and_symmetric():
    x = np.sort(np.concatenate([-_sweep(90.0, 1021), _sweep(90.0, 1021)]))
    s = O.sigmoid_f32(x)
    assert np.all(np.diff(s.astype(np.float64)) >= 0)
    assert O.sigmoid_f32(F32(0.0)) == F32(0.5) and O.sigmoid_f32(F32(-0.0)) == F32(0.5)
    xs = np.linspace(-20, 20, 4001, dtype=F32)
    assert np.max(np.abs(O.sigmoid_f32(xs).astype(np.float64) + O.sigmoid_f32(-xs) - 1.0)) < 2e-7


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.integers(-6, 6, 200000),
                        [0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-30]]).astype(F32)
    # exact ties between two bf16 neighbours: both directions of round-to-even
    base = (rng.integers(0x3F000000, 0x40000000, 1000) & ~0xFFFF).astype(np.uint32)
    ties = (base | 0x8000).view(F32)
    v = np.concatenate([v, ties])
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(O.bf16_round(v), ref)


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    d = O.e4m3_decode(codes)
    t = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    both_nan = np.isnan(d) & np.isnan(t)
    assert np.all(both_nan | (d == t))
    # closed-form anchors of the format
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0       # largest finite
    assert d[0x01] == 2.0 ** -9                          # smallest subnormal
    assert d[0x08] == 2.0 ** -6                          # smallest normal
    assert d[0x38] == 1.0 and np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.sum(np.isnan(d)) == 2


def test_e4m3_round_matches_torch_and_round_trips():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(300000) * 10.0 ** rng.uniform(-4, 2.6, 300000)).astype(F32)
    v = v[np.abs(v) < 464.0]       # torch's cast is non-saturating above this
    ref = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(O.e4m3_round(v), ref.astype(np.float64))
    vals = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = vals[np.isfinite(vals)]
    assert np.array_equal(O.e4m3_round(fin), fin)


def test_e4m3_round_ties_to_even_and_saturates():
    # 1.0 (code 0x38, even) and 1.125 (0x39, odd): the midpoint goes to 1.0
    assert O.e4m3_round(1.0625) == 1.0
    # 1.125 (odd) and 1.25 (even): midpoint 1.1875 goes to 1.25
    assert O.e4m3_round(1.1875) == 1.25
    # subnormal spacing 2**-9: midpoint of 1*2**-9 and 2*2**-9 goes to 2*2**-9
    assert O.e4m3_round(1.5 * 2.0 ** -9) == 2.0 * 2.0 ** -9
    assert O.e4m3_round(0.5 * 2.0 ** -9) == 0.0
    assert O.e4m3_round(1e6) == 448.0 and O.e4m3_round(-500.0) == -448.0


def test_quantize_fp8_rows_invariants():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((16, 512)).astype(F32)
    v[3, 128:256] = 0.0
    q, s = O.quantize_fp8_rows(v)
    assert s.shape == (16, 4) and s.dtype == F32
    assert np.all(np.abs(q) <= 448.0)
    # the element of largest magnitude in each block maps to +-448
    blk = q.reshape(16, 4, 128)
    amax = np.max(np.abs(blk), axis=2)
    assert np.all((amax == 448.0) | (s == 1.0))
    assert s[3, 1] == 1.0 and np.all(blk[3, 1] == 0.0)
    # every quantised value is an e4m3 value
    assert np.array_equal(O.e4m3_round(q), q)
    # dequantisation error is within half an e4m3 step (relative 2**-4)
    deq = (blk * s[:, :, None]).reshape(16, 512)
    err = np.abs(deq - v)
    assert np.all(err <= np.maximum(np.abs(v) * 2.0 ** -4, (s.repeat(128, axis=1)) * 2.0 ** -10) + 1e-12)


def test_quantize_fp8_rows_matches_torch_cast_and_tiny_blocks():
    """Ordinary blocks: the codes are torch's own float8_e4m3fn cast of the
    float32 product v * (448 / a) (an independent RNE implementation); a
    block whose 448 / a overflows float32 keeps finite codes."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal((8, 256)).astype(F32) * rng.uniform(1e-3, 1e3, (8, 1)).astype(F32)
    q, s = O.quantize_fp8_rows(v)
    a = np.max(np.abs(v.reshape(8, 2, 128)), axis=2)
    inv = torch.from_numpy(np.full_like(a, 448.0)) / torch.from_numpy(a)
    prod = torch.from_numpy(v.reshape(8, 2, 128)) * inv[:, :, None]
    want = prod.to(torch.float8_e4m3fn).double().reshape(8, 256).numpy()
    assert np.array_equal(q, want)
    assert np.array_equal(s, (torch.from_numpy(a) / 448.0).numpy())
    tiny = np.zeros((1, 128), F32)
    tiny[0, :] = F32(2.0 ** -130)
    tiny[0, 1] = F32(-(2.0 ** -131))
    qt, st = O.quantize_fp8_rows(tiny)
    assert np.all(np.isfinite(qt)) and np.all(np.abs(qt) <= 448.0)
    # inv = largest float32 ~ 2**128: 2**-130 -> 0.25, -2**-131 -> -0.125
    assert qt[0, 0] == 0.25 and qt[0, 1] == -0.125
    assert st[0, 0] == F32(2.0 ** -130) / F32(448.0)


def test_block_weight_dequant_matches_torch():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, (256, 384), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0       # no NaN codes
    scales = rng.uniform(0.001, 0.01, (2, 3)).astype(F32)
    got = O.dequant_block_weight(codes, scales)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).double()
    ts = torch.from_numpy(scales).double().repeat_interleave(128, 0).repeat_interleave(128, 1)
    assert np.array_equal(got, (t * ts).numpy())
