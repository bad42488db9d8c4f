"""Pins of the oracle's logits over a paged quantized key cache
(oracle.indexer_logits_paged / paged_keys) against things other than itself:

* fp8 keys: scattering dense fp8 keys into a block-permuted cache must give
  exactly the dense fp8 logits (an already-pinned routine);
* mxfp4 keys: an integer/dyadic-exact brute force in Fractions with explicit
  loops over heads, dims, nibbles and the block table;
* mxfp4 keys: the gather oracle's bf16 rows (exact here) fed to the dense
  bf16 logits must give exactly the paged logits;
* invariants: an E8M0 0xFF group equals a zeroed group, one more scale step
  doubles a key's score, block permutation leaves logits unchanged.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

E2M1_TABLE = [Fraction(v) for v in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]


def _e2m1_frac(nib):
    v = E2M1_TABLE[nib & 7]
    return -v if nib & 8 else v


def _e4m3_frac_of_small(code):
    """Exact value of an e4m3 code known to be a normal number."""
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    assert 0 < e < 15
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def _random_table(rng, B, MB, NB):
    perm = rng.permutation(NB).astype(np.int32)
    return perm[: B * MB].reshape(B, MB)


def test_paged_fp8_equals_dense_fp8_through_permuted_blocks():
    rng = np.random.default_rng(11)
    B, T, H, D, K, bs = 2, 3, 64, 128, 40, 8
    MB = K // bs
    q8 = rng.integers(0, 0x7E, size=(B, T, H, D), dtype=np.uint8)  # no NaN codes
    q8 |= rng.integers(0, 2, size=q8.shape, dtype=np.uint8) << 7
    k8 = rng.integers(0, 0x7E, size=(B, K, D), dtype=np.uint8)
    sq = rng.uniform(0.01, 0.1, size=(B, T, H)).astype(np.float32)
    sk = rng.uniform(0.01, 0.1, size=(B, K)).astype(np.float32)
    w = rng.standard_normal((B, T, H)).astype(np.float32)
    limit = np.array([[39, 17, 0], [25, -1, 60]], dtype=np.int32)
    dense = oracle.indexer_logits(q8, k8, w, limit, sq, sk, "fp8")

    NB = B * MB + 3
    table = _random_table(rng, B, MB, NB)
    cache = np.zeros((NB, bs, D), dtype=np.uint8)
    cscale = np.zeros((NB, bs), dtype=np.float32)
    for b in range(B):
        for j in range(K):
            cache[table[b, j // bs], j % bs] = k8[b, j]
            cscale[table[b, j // bs], j % bs] = sk[b, j]
    paged = oracle.indexer_logits_paged(q8, sq, w, limit, cache, cscale, table, bs, K, "fp8")
    assert np.array_equal(paged, dense, equal_nan=True)


def _mxfp4_case(rng, B, T, H, D, K, bs, scale_bytes):
    MB = (K + bs - 1) // bs
    NB = B * MB + 2
    table = _random_table(rng, B, MB, NB)
    kc = rng.integers(0, 256, size=(NB, bs, D // 2), dtype=np.uint8)
    ks = rng.choice(np.array(scale_bytes, dtype=np.uint8), size=(NB, bs, D // 32))
    return kc, ks, table


def test_paged_mxfp4_exact_brute_force():
    rng = np.random.default_rng(5)
    B, T, H, D, K, bs = 2, 2, 3, 64, 10, 4
    kc, ks, table = _mxfp4_case(rng, B, T, H, D, K, bs, [125, 126, 127, 128, 129, 0xFF])
    # q codes: normal e4m3 numbers with exponent field 5..9 (values 1/4 .. 4ish)
    q8 = (rng.integers(5, 10, size=(B, T, H, D)) << 3 | rng.integers(0, 8, size=(B, T, H, D))).astype(np.uint8)
    q8 |= (rng.integers(0, 2, size=q8.shape) << 7).astype(np.uint8)
    sq = np.float32(2.0) ** rng.integers(-3, 3, size=(B, T, H)).astype(np.float32)
    wm = rng.integers(-8, 9, size=(B, T, H))
    w = (wm / 8.0).astype(np.float32)
    limit = np.array([[9, 4], [0, -1]], dtype=np.int32)
    got = oracle.indexer_logits_paged(q8, sq, w, limit, kc, ks, table, bs, K, "mxfp4")
    for b in range(B):
        for t in range(T):
            for j in range(K):
                if j > limit[b, t]:
                    assert got[b, t, j] == -np.inf
                    continue
                blk, off = int(table[b, j // bs]), j % bs
                total = Fraction(0)
                for h in range(H):
                    dot = Fraction(0)
                    for d in range(D):
                        byte = int(kc[blk, off, d // 2])
                        nib = byte & 0xF if d % 2 == 0 else byte >> 4
                        sb = int(ks[blk, off, d // 32])
                        scale = Fraction(0) if sb == 0xFF else Fraction(2) ** (sb - 127)
                        qv = _e4m3_frac_of_small(int(q8[b, t, h, d])) * Fraction(float(sq[b, t, h]))
                        dot += qv * _e2m1_frac(nib) * scale
                    total += Fraction(int(wm[b, t, h]), 8) * max(dot, Fraction(0))
                assert got[b, t, j] == np.float32(float(total)), (b, t, j)


def test_paged_mxfp4_matches_gather_then_dense_bf16():
    rng = np.random.default_rng(9)
    B, T, H, D, K, bs = 2, 3, 64, 128, 70, 16
    kc, ks, table = _mxfp4_case(rng, B, T, H, D, K, bs, list(range(118, 137)) + [0xFF])
    q8 = rng.integers(0, 0x7E, size=(B, T, H, D), dtype=np.uint8)
    q8 |= rng.integers(0, 2, size=q8.shape, dtype=np.uint8) << 7
    sq = np.float32(2.0) ** rng.integers(-6, 0, size=(B, T, H)).astype(np.float32)
    w = rng.standard_normal((B, T, H)).astype(np.float32)
    limit = np.array([[69, 30, 5], [64, 63, 0]], dtype=np.int32)
    paged = oracle.indexer_logits_paged(q8, sq, w, limit, kc, ks, table, bs, K, "mxfp4")
    # dense keys: the gather of every position (exact in bf16 for these scales)
    sel = np.tile(np.arange(K, dtype=np.int32), (B, 1))
    k_bits = oracle.mxfp4_paged_gather(kc, ks, table, sel, np.arange(B, dtype=np.int32), bs)
    # q = e4m3 * 2^m is exact in bf16 (3 mantissa bits)
    qf = torch.from_numpy(q8).view(torch.float8_e4m3fn).float() * torch.from_numpy(sq)[..., None]
    q_bits = qf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f64(q_bits),
                          oracle.e4m3_to_f64(q8) * sq.astype(np.float64)[..., None])
    dense = oracle.indexer_logits(q_bits, k_bits, w, limit, dtype="bf16")
    assert np.array_equal(paged, dense, equal_nan=True)


def _one_key_case(seed):
    rng = np.random.default_rng(seed)
    B, T, H, D, K, bs = 1, 2, 64, 128, 8, 4
    kc, ks, table = _mxfp4_case(rng, B, T, H, D, K, bs, [124, 126, 127, 130])
    q8 = rng.integers(0, 0x7E, size=(B, T, H, D), dtype=np.uint8)
    sq = rng.uniform(0.01, 0.1, size=(B, T, H)).astype(np.float32)
    w = rng.uniform(0.0, 1.0, size=(B, T, H)).astype(np.float32)
    limit = np.full((B, T), K - 1, dtype=np.int32)
    return dict(q=q8, q_scale=sq, w=w, limit=limit, k_cache=kc, k_scale=ks, block_table=table,
                block_size=bs, K=K, kfmt="mxfp4")


def test_paged_mxfp4_ff_group_equals_zeroed_group():
    c = _one_key_case(3)
    j, g = 5, 2
    blk, off = int(c["block_table"][0, j // 4]), j % 4
    a = dict(c, k_scale=c["k_scale"].copy())
    a["k_scale"][blk, off, g] = 0xFF
    z = dict(c, k_cache=c["k_cache"].copy())
    z["k_cache"][blk, off, 16 * g: 16 * g + 16] = 0      # the group's 32 nibbles -> +0
    assert np.array_equal(oracle.indexer_logits_paged(**a), oracle.indexer_logits_paged(**z))


def test_paged_mxfp4_scale_step_doubles_a_key():
    c = _one_key_case(4)
    j = 6
    blk, off = int(c["block_table"][0, j // 4]), j % 4
    base = oracle.indexer_logits_paged(**c)
    up = dict(c, k_scale=c["k_scale"].copy())
    up["k_scale"][blk, off] += 1
    got = oracle.indexer_logits_paged(**up)
    assert np.array_equal(got[..., j], 2 * base[..., j])
    others = [i for i in range(c["K"]) if i != j]
    assert np.array_equal(got[..., others], base[..., others])


def test_paged_block_permutation_invariance():
    c = _one_key_case(8)
    rng = np.random.default_rng(1)
    NB = c["k_cache"].shape[0]
    perm = rng.permutation(NB)
    inv = np.argsort(perm)
    moved = dict(c, k_cache=c["k_cache"][perm], k_scale=c["k_scale"][perm],
                 block_table=inv[c["block_table"]].astype(np.int32))
    assert np.array_equal(oracle.indexer_logits_paged(**moved), oracle.indexer_logits_paged(**c))


@pytest.mark.parametrize("kfmt", ["mxfp4", "fp8"])
def test_paged_keys_reads_only_through_the_table(kfmt):
    rng = np.random.default_rng(2)
    NB, bs, D = 6, 4, 128
    if kfmt == "mxfp4":
        kc = rng.integers(0, 256, size=(NB, bs, D // 2), dtype=np.uint8)
        ks = rng.integers(120, 134, size=(NB, bs, D // 32), dtype=np.uint8)
    else:
        kc = rng.integers(0, 0x7E, size=(NB, bs, D), dtype=np.uint8)
        ks = rng.uniform(0.5, 2.0, size=(NB, bs)).astype(np.float32)
    table = np.array([[4, 1, 5]], dtype=np.int32)
    keys = oracle.paged_keys(kc, ks, table, 0, 10, bs, kfmt)
    # block 4 holds positions 0..3, block 1 positions 4..7, block 5 positions 8..9
    for p, (blk, off) in enumerate([(4, 0), (4, 1), (4, 2), (4, 3), (1, 0), (1, 1), (1, 2), (1, 3),
                                    (5, 0), (5, 1)]):
        one = oracle.paged_keys(kc, ks, np.array([[blk]], dtype=np.int32), 0, off + 1, bs, kfmt)[off]
        assert np.array_equal(keys[p], one)
