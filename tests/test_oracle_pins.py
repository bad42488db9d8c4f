"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a closed form, a different algorithm
(brute force), an independent decoder (torch's float8 / bfloat16 casts) or
hand-derived bytes under tests/golden/, chosen so that a plausible slip in the
oracle (dropped relu, relu after the head sum, wrong sign, swapped t/j, wrong
head weight, off-by-one causal mask, wrong nibble order, wrong group scale,
unstable tie order) fails at least one of them.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import indexer as oi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits_of_small_ints(a):
    """bf16 bits of small integers, built from the IEEE layout by hand."""
    a = np.asarray(a, dtype=np.int64)
    out = np.zeros(a.shape, dtype=np.uint16)
    for idx, v in np.ndenumerate(a):
        if v == 0:
            continue
        m = abs(int(v))
        e = m.bit_length() - 1                       # m = 1.f * 2**e
        frac = (m - (1 << e)) << (7 - e)             # 7 stored mantissa bits (m < 256)
        out[idx] = ((127 + e) << 7) | frac | (0x8000 if v < 0 else 0)
    return out


# ----------------------------------------------------------------------------- formats
def test_e4m3_all_codes_match_torch_decoder():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.isnan(mine).sum() == 2                 # 0x7F and 0xFF only
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0
    assert mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6 and mine[0x38] == 1.0


def test_e8m0_matches_torch_except_ff():
    b = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(oracle.e8m0_to_f64(b), ref)
    assert oracle.e8m0_to_f64(np.uint8(0xFF)) == 0.0     # the gather's 0xFF -> 0 rule


def test_e2m1_table():
    # OCP MX E2M1 magnitudes for codes 0..7; 8..15 negate them (8 is -0.0)
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = oracle.e2m1_to_f64(np.arange(16))
    assert list(got[:8]) == mags
    assert list(-got[8:]) == mags
    assert np.signbit(got[8]) and not np.signbit(got[0])


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]           # drop inf/NaN
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), ref)


def test_bf16_rounding_matches_torch_single_rounding():
    rng = np.random.default_rng(6)
    # float32-representable values across the whole range (incl. subnormals): one RNE step
    f32 = rng.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    f32 = f32[np.isfinite(f32)]
    f32 = np.concatenate([f32, np.float32([0.0, -0.0, 3.3895314e38, -3.3895314e38,
                                            1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8])])
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = oracle.f64_to_bf16_bits(f32.astype(np.float64))
    assert np.array_equal(mine, ref)
    assert oracle.f64_to_bf16_bits(2.0 ** 128) == 0x7F80
    assert oracle.f64_to_bf16_bits(-(2.0 ** 130)) == 0xFF80


def test_small_int_bf16_builder_agrees_with_torch():
    a = np.arange(-255, 256)
    ref = torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(bf16_bits_of_small_ints(a), ref.view(np.uint16))


# ----------------------------------------------------------------------------- logits
def _exact_logits(qi, ki, w_frac, limit):
    """Exact rational logits for integer q/k by Python integers (brute force)."""
    T, H, D = qi.shape
    K = ki.shape[0]
    out = np.empty((T, K), dtype=object)
    for t in range(T):
        for j in range(K):
            if j > limit[t]:
                out[t, j] = None
                continue
            s = Fraction(0)
            for h in range(H):
                dot = int(sum(int(qi[t, h, d]) * int(ki[j, d]) for d in range(D)))
                s += w_frac[t][h] * max(dot, 0)
            out[t, j] = s
    return out


def test_logits_integer_exact_brute_force():
    rng = np.random.default_rng(11)
    T, K, H, D = 3, 7, 4, 6
    qi = rng.integers(-3, 4, size=(1, T, H, D))
    ki = rng.integers(-3, 4, size=(1, K, D))
    wm = rng.integers(-8, 9, size=(1, T, H))
    w = (wm / 8.0).astype(np.float32)
    limit = np.array([[6, 2, 0]], dtype=np.int32)
    got = oracle.indexer_logits(bf16_bits_of_small_ints(qi), bf16_bits_of_small_ints(ki), w, limit)
    ref = _exact_logits(qi[0], ki[0], [[Fraction(int(m), 8) for m in row] for row in wm[0]], limit[0])
    for t in range(T):
        for j in range(K):
            if ref[t, j] is None:
                assert got[0, t, j] == -np.inf
            else:
                assert Fraction(float(got[0, t, j])) == ref[t, j]


def test_logits_rank1_closed_form():
    """q[t,h] = a[t,h] u, k[j] = c[j] u  =>  dot = a c |u|^2, and the relu picks a sign."""
    rng = np.random.default_rng(12)
    T, K, H, D = 5, 9, 64, 128
    u = rng.integers(-1, 3, size=D)
    U = int((u * u).sum())
    a = rng.integers(-3, 4, size=(T, H))
    c = rng.integers(-3, 4, size=K)
    wm = rng.integers(-8, 9, size=(T, H))
    q = bf16_bits_of_small_ints(a[:, :, None] * u[None, None, :])[None]
    k = bf16_bits_of_small_ints(c[:, None] * u[None, :])[None]
    w = (wm / 8.0).astype(np.float32)[None]
    got = oracle.indexer_logits(q, k, w)[0]
    pos = (wm * np.maximum(a, 0)).sum(1) / 8.0     # [T]: sum_h w max(a,0)
    neg = (wm * np.maximum(-a, 0)).sum(1) / 8.0    # [T]: sum_h w max(-a,0)
    exp = np.where(c[None, :] >= 0, c[None, :] * U * pos[:, None], -c[None, :] * U * neg[:, None])
    assert np.array_equal(got, exp.astype(np.float32))
    assert np.any(got != 0)


@pytest.mark.parametrize("limits", [[-1, 0, 5, 40], [39, 100, -7, 20]])
def test_logits_mask_is_inclusive_and_exact_minus_inf(limits):
    rng = np.random.default_rng(13)
    T, K = 4, 40
    q = bf16_bits_of_small_ints(rng.integers(-2, 3, size=(1, T, 64, 128)))
    k = bf16_bits_of_small_ints(rng.integers(-2, 3, size=(1, K, 128)))
    w = np.abs(rng.standard_normal((1, T, 64))).astype(np.float32)
    lim = np.array([limits], dtype=np.int32)
    got = oracle.indexer_logits(q, k, w, lim)[0]
    for t in range(T):
        n = max(0, min(limits[t] + 1, K))
        assert np.all(np.isfinite(got[t, :n]))
        assert np.all(got[t, n:] == -np.inf)


def _rand_bf16(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_logits_invariants():
    rng = np.random.default_rng(14)
    T, K, H, D = 3, 33, 64, 128
    q = _rand_bf16(rng, (1, T, H, D))
    k = _rand_bf16(rng, (1, K, D))
    w = (rng.standard_normal((1, T, H)) / 8).astype(np.float32)
    base = oracle.indexer_logits(q, k, w)
    # w >= 0  =>  every score >= 0 (each head term is a relu)
    assert np.all(oracle.indexer_logits(q, k, np.abs(w)) >= 0)
    # permuting heads of q and w together changes nothing
    perm = rng.permutation(H)
    permuted = oracle.indexer_logits(q[:, :, perm], k, w[:, :, perm])
    np.testing.assert_allclose(permuted, base, rtol=1e-6, atol=1e-6)
    # q -> 2q (exact in bf16) doubles every score exactly
    q2 = (q.astype(np.uint32) + (1 << 7)).astype(np.uint16)    # exponent + 1
    q2[(q & 0x7FFF) == 0] = q[(q & 0x7FFF) == 0]
    assert np.array_equal(oracle.indexer_logits(q2, k, w), 2 * base)
    # linear in w
    w2 = (rng.standard_normal((1, T, H)) / 8).astype(np.float32)
    np.testing.assert_allclose(oracle.indexer_logits(q, k, w + w2),
                               base + oracle.indexer_logits(q, k, w2), rtol=1e-5, atol=1e-4)
    # only positive dots contribute: flipping k's sign swaps which heads count
    neg = oracle.indexer_logits(q, (k ^ np.uint16(0x8000)), w)
    q_hat = oracle.bf16_bits_to_f64(q)[0]
    k_hat = oracle.bf16_bits_to_f64(k)[0]
    dots = np.einsum("thd,jd->thj", q_hat, k_hat)
    exp_neg = (w[0][:, :, None] * np.maximum(-dots, 0)).sum(1)
    np.testing.assert_allclose(neg[0], exp_neg.astype(np.float32), rtol=1e-6, atol=1e-5)


def test_logits_fp8_agrees_with_bf16_on_shared_values():
    """Values representable in both e4m3 and bf16 give the same scores (scale 1)."""
    rng = np.random.default_rng(16)
    T, K, H, D = 2, 11, 64, 128
    ints = np.arange(-15, 16)
    qi = rng.choice(ints, size=(1, T, H, D))
    ki = rng.choice(ints, size=(1, K, D))
    codes = torch.tensor(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()
    to_code = {float(v): c for c, v in enumerate(codes) if np.isfinite(v)}
    q8 = np.vectorize(lambda v: to_code[float(v)])(qi).astype(np.uint8)
    k8 = np.vectorize(lambda v: to_code[float(v)])(ki).astype(np.uint8)
    w = (rng.standard_normal((1, T, H)) / 8).astype(np.float32)
    a = oracle.indexer_logits(q8, k8, w, q_scale=np.ones((1, T, H), np.float32),
                              k_scale=np.ones((1, K), np.float32), dtype="fp8")
    b = oracle.indexer_logits(bf16_bits_of_small_ints(qi), bf16_bits_of_small_ints(ki), w)
    assert np.array_equal(a, b)
    # a power-of-two scale on q scales every score by it
    c = oracle.indexer_logits(q8, k8, w, q_scale=np.full((1, T, H), 0.25, np.float32),
                              k_scale=np.ones((1, K), np.float32), dtype="fp8")
    assert np.array_equal(c, b * np.float32(0.25))


# ----------------------------------------------------------------------------- top-k
def _topk_brute(scores, n, k):
    """Repeated arg-max over unselected j, scanning j upward with strict '>'."""
    vals = [0.0 if float(x) == 0.0 else float(x) for x in scores[:n]]
    taken = [False] * n
    out = []
    for _ in range(min(k, n)):
        best = -1
        for j in range(n):
            if not taken[j] and (best < 0 or vals[j] > vals[best]):
                best = j
        taken[best] = True
        out.append(best)
    return out + [-1] * (k - len(out))


@pytest.mark.parametrize("seed", range(6))
def test_topk_against_brute_force_with_heavy_ties(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(25):
        K = int(rng.integers(1, 60))
        k = int(rng.choice([1, 2, 4, 16]))
        n = int(rng.integers(0, K + 1))
        row = rng.choice(np.float32([0.0, -0.0, 1.0, 2.0, -1.0, np.inf, -np.inf]), size=K)
        assert list(oracle.topk_row(row, n, k)) == _topk_brute(row, n, k)


def test_topk_closed_forms():
    n, k = 50, 16
    assert list(oracle.topk_row(np.full(n, 3.0, np.float32), n, k)) == list(range(k))
    assert list(oracle.topk_row(-np.arange(n, dtype=np.float32), n, k)) == list(range(k))
    assert list(oracle.topk_row(np.arange(n, dtype=np.float32), n, k)) == list(range(n - 1, n - 1 - k, -1))
    assert list(oracle.topk_row(np.arange(n, dtype=np.float32), 5, k)) == [4, 3, 2, 1, 0] + [-1] * 11
    assert list(oracle.topk_row(np.ones(n, np.float32), 0, 4)) == [-1] * 4
    assert list(oracle.topk_row(np.float32([-0.0, 0.0]), 2, 1)) == [0]
    assert list(oracle.topk_row(np.float32([0.0, -0.0]), 2, 1)) == [0]
    # keys past n are never chosen, however large
    assert list(oracle.topk_row(np.float32([1, 2, 3, 99, 99]), 3, 3)) == [2, 1, 0]


def test_topk_invariants_random_rows():
    rng = np.random.default_rng(7)
    K, k = 3000, 512
    x = rng.standard_normal((6, K)).astype(np.float32)
    x[3, ::7] = x[3, 0]                                # inject ties
    lim = np.array([K - 1, 100, 511, 2999, -1, 512], dtype=np.int32)
    idx = oracle.indexer_topk(x, lim, k)
    for r in range(6):
        n = max(0, min(lim[r] + 1, K))
        m = min(k, n)
        sel = idx[r, :m]
        assert np.all(idx[r, m:] == -1) and np.all(sel >= 0) and np.all(sel < n)
        assert len(set(sel.tolist())) == m
        if m:
            rest = np.setdiff1d(np.arange(n), sel)
            if rest.size:
                assert x[r, sel].min() >= x[r, rest].max()
            s = x[r, sel]
            assert np.all((s[:-1] > s[1:]) | ((s[:-1] == s[1:]) & (sel[:-1] < sel[1:])))


# ----------------------------------------------------------------------------- gather
def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "mxfp4_hand_rows.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            p, s, lo, hi = (int(t, 16) for t in line.split()[:4])
            rows.append((p, s, lo, hi))
    return rows


def test_gather_hand_built_golden_bytes():
    rows = _golden_rows()
    bs = 16
    fp4 = np.zeros((1, bs, 64), np.uint8)
    sc = np.full((1, bs, 4), 127, np.uint8)
    for i, (p, s, _, _) in enumerate(rows):
        fp4[0, i, :] = p
        sc[0, i, :] = s
    sel = np.array([list(range(len(rows)))], dtype=np.int32)
    out = oracle.mxfp4_paged_gather(fp4, sc, np.zeros((1, 1), np.int32), sel,
                                    np.zeros(1, np.int32), bs)
    for i, (_, _, lo, hi) in enumerate(rows):
        assert np.all(out[0, i, 0::2] == lo), i
        assert np.all(out[0, i, 1::2] == hi), i


def test_gather_group_scales_and_nibble_order():
    fp4 = np.full((1, 4, 64), 0x42, np.uint8)           # low 2 -> 1.0, high 4 -> 2.0
    sc = np.array([[[127, 128, 129, 255]] * 4], np.uint8)
    out = oracle.mxfp4_paged_gather(fp4, sc, np.zeros((1, 1), np.int32),
                                    np.array([[2]], np.int32), np.zeros(1, np.int32), 4)
    vals = oracle.bf16_bits_to_f64(out[0, 0])
    exp = np.concatenate([np.tile([1.0, 2.0], 16) * s for s in (1.0, 2.0, 4.0, 0.0)])
    assert np.array_equal(vals, exp)


def test_gather_negative_slots_zero_and_block_permutation_invariance():
    rng = np.random.default_rng(21)
    NB, bs = 8, 64
    fp4 = rng.integers(0, 256, size=(NB, bs, 64), dtype=np.uint8)
    sc = rng.integers(118, 137, size=(NB, bs, 4), dtype=np.uint8)
    table = rng.permutation(NB).astype(np.int32).reshape(2, 4)
    sel = rng.integers(-3, 256, size=(4, 32)).astype(np.int32)
    row_seq = np.array([0, 1, 1, 0], np.int32)
    out = oracle.mxfp4_paged_gather(fp4, sc, table, sel, row_seq, bs)
    assert np.all(out[sel < 0] == 0)
    # relabel physical blocks: move block b to pi[b], and the table with it
    pi = rng.permutation(NB)
    fp4_p = np.empty_like(fp4); fp4_p[pi] = fp4
    sc_p = np.empty_like(sc); sc_p[pi] = sc
    out_p = oracle.mxfp4_paged_gather(fp4_p, sc_p, pi[table].astype(np.int32), sel, row_seq, bs)
    assert np.array_equal(out, out_p)
    # element d of slot (r,s): direct re-derivation for a few samples
    for (r, s) in [(0, 0), (1, 5), (3, 31)]:
        p = sel[r, s]
        if p < 0:
            continue
        blk, off = table[row_seq[r], p // bs], p % bs
        for d in (0, 1, 63, 64, 127):
            nib = (fp4[blk, off, d // 2] >> (4 * (d % 2))) & 0xF
            v = oracle.e2m1_to_f64(nib) * oracle.e8m0_to_f64(sc[blk, off, d // 32])
            assert oracle.bf16_bits_to_f64(out[r, s, d]) == v
