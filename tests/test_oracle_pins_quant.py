"""Pins of the oracle's producers (oracle/quant.py) against things other than
themselves: torch's float8_e4m3fn cast (a library routine), hand-derived
E2M1 rounding boundaries and E8M0 exponents, round trips through the pinned
decoders, the gather oracle, and error bounds."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 50,
        rng.uniform(-2 ** -6, 2 ** -6, 5000).astype(np.float32),       # subnormal range
        oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8)).astype(np.float32),  # exact codes
    ])
    # exact midpoints between neighbouring codes (ties go to the even code)
    pos = np.sort(oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8)))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids]).astype(np.float32)
    v = np.clip(v, -448, 448)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = quant.e4m3_encode(v)
    same = (got == ref) | ((got & 0x7F) == 0) & ((ref & 0x7F) == 0)   # +-0 both fine
    assert same.all(), v[~same][:10]


def test_e2m1_encode_boundaries_and_round_trip():
    # hand-derived: representable 0, .5, 1, 1.5, 2, 3, 4, 6; midpoints tie to the even code
    cases = {0.0: 0.0, 0.24: 0.0, 0.25: 0.0, 0.26: 0.5, 0.75: 1.0, 1.25: 1.0, 1.26: 1.5,
             1.75: 2.0, 2.5: 2.0, 2.6: 3.0, 3.5: 4.0, 5.0: 4.0, 5.01: 6.0, 7.0: 6.0, 1e9: 6.0}
    for x, want in cases.items():
        assert oracle.e2m1_to_f64(quant.e2m1_encode(x)) == want, x
        assert oracle.e2m1_to_f64(quant.e2m1_encode(-x)) == -want, -x
    codes = np.arange(16)
    assert np.array_equal(quant.e2m1_encode(oracle.e2m1_to_f64(codes))[codes != 8], codes[codes != 8])
    # monotone, and within half the local gap
    v = np.linspace(-7, 7, 20001)
    d = oracle.e2m1_to_f64(quant.e2m1_encode(v))
    assert np.all(np.diff(d) >= 0)
    inside = np.abs(v) <= 6
    gap = np.where(np.abs(v) < 2, 0.5, np.where(np.abs(v) < 4, 1.0, 2.0))
    assert np.all(np.abs(d - v)[inside] <= gap[inside] / 2 + 1e-12)


def test_quant_fp8_rows_scale_and_codes():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 128)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32)
    x[3] = 0
    codes, scale = quant.quant_fp8_rows(x)
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(scale[amax > 0], (amax[amax > 0] / np.float32(448)).astype(np.float32))
    assert scale[3] == 1.0 and np.all(codes[3] & 0x7F == 0)
    # the largest element of every row lands on +-448
    top = np.abs(x).argmax(axis=1)
    assert np.all((codes[np.arange(64), top] & 0x7F)[amax > 0] == 0x7E)
    ref = torch.from_numpy(x / scale[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    # dequantized rows within half an e4m3 step (relative 2^-4) of x, plus the subnormal quantum
    back = oracle.e4m3_to_f64(codes) * scale[:, None]
    assert np.all(np.abs(back - x) <= np.abs(x) * 2 ** -4 + scale[:, None] * 2 ** -10)


def test_mxfp4_encode_scale_rule():
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, 0:32] = np.linspace(-6, 6, 32)           # amax 6: floor(log2 6) = 2 -> e 0 -> byte 127
    x[0, 32:64] = 1.0                              # amax 1: e -2 -> byte 125, elements 4.0
    x[0, 64:96] = 0.0                              # all zero -> byte 0, nibbles 0
    x[0, 96] = 7.9                                 # amax 7.9: e 0; 7.9 saturates to 6
    x[0, 97] = -0.3
    packed, sc = quant.mxfp4_encode_rows(x)
    assert sc.tolist() == [[127, 125, 0, 127]]
    nib = np.empty(128, dtype=np.int64)
    nib[0::2], nib[1::2] = packed[0] & 0xF, packed[0] >> 4
    vals = oracle.e2m1_to_f64(nib)
    assert np.all(vals[32:64] == 4.0)
    assert np.all(nib[64:96] == 0)
    assert vals[96] == 6.0 and vals[97] == -0.5 and np.all(vals[98:128] == 0)
    assert vals[0] == -6.0 and vals[31] == 6.0


def test_mxfp4_write_then_gather_round_trip():
    rng = np.random.default_rng(2)
    N, NB, bs = 40, 8, 16
    x = (rng.standard_normal((N, 128)) * np.exp2(rng.integers(-8, 8, (N, 1)))).astype(np.float32)
    slots = rng.permutation(NB * bs)[:N].astype(np.int64)
    slots[5] = -1                                   # skipped row
    kv0 = np.zeros((NB, bs, 64), dtype=np.uint8)
    sc0 = np.zeros((NB, bs, 4), dtype=np.uint8)
    kv, sc = quant.mxfp4_cache_write(x, slots, kv0, sc0)
    # reading every written slot back through the gather oracle (identity table)
    table = np.arange(NB, dtype=np.int32)[None, :]
    sel = np.where(slots >= 0, slots, -1)[None, :].astype(np.int32)
    back = oracle.bf16_bits_to_f64(oracle.mxfp4_paged_gather(kv, sc, table, sel, np.zeros(1, np.int32), bs))[0]
    ok = slots >= 0
    # error bound: half the E2M1 step at each element's magnitude, times the
    # group scale; above 6 (the group exponent puts amax in [4, 8)) the
    # element saturates and the error is exactly the excess over 6
    e = sc.astype(np.int64)[slots[ok] // bs, slots[ok] % bs] - 127          # [n, 4]
    step = np.repeat(np.exp2(e.astype(np.float64)), 32, axis=1)              # scale per element
    mag = np.abs(x[ok]) / step
    assert np.all(mag < 8)
    half_gap = np.where(mag < 2, 0.25, np.where(mag < 4, 0.5, 1.0)) * step
    err = np.abs(back[ok] - x[ok])
    sat = mag > 6
    assert np.all(err[~sat] <= half_gap[~sat] + 1e-30)
    assert np.allclose(err[sat], (mag[sat] - 6) * step[sat], rtol=1e-6)
    assert np.all(back[~ok] == 0)
    # untouched slots stay zero
    written = np.zeros(NB * bs, dtype=bool)
    written[slots[ok]] = True
    assert np.all(kv.reshape(NB * bs, 64)[~written] == 0)
    # values already on the grid come back exactly
    g = oracle.e2m1_to_f64(rng.integers(0, 16, (4, 128))) * 2.0 ** 3
    g[:, ::32] = 6 * 2.0 ** 3                       # make every group's amax a grid value
    kv2, sc2 = quant.mxfp4_cache_write(g.astype(np.float32), np.arange(4), kv0, sc0)
    back2 = oracle.bf16_bits_to_f64(oracle.mxfp4_paged_gather(
        kv2, sc2, table, np.arange(4, dtype=np.int32)[None, :], np.zeros(1, np.int32), bs))[0]
    assert np.array_equal(back2, g)
