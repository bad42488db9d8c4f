"""Pins of the oracle's sparse attention (oracle/attention.py) against things
other than itself: torch's scaled_dot_product_attention (a library routine;
the sink becomes one more key, of value 0, whose additive mask is the sink
logit), closed forms (all scores equal), limits (a dominant key, no valid
slot), invariances (slot order, padding slots) and the composition with the
pinned gather oracle."""
import numpy as np
import torch

import oracle
from oracle.attention import sparse_attention


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _case(seed, R=3, H=4, k=9, D=16, qs=0.3):
    rng = np.random.default_rng(seed)
    q = _bf16(rng.standard_normal((R, H, D)) * qs)
    v = _bf16(rng.standard_normal((R, k, D)))
    sel = rng.integers(0, 50, (R, k)).astype(np.int32)
    sel[0, 2] = -1
    sel[1, ::3] = -1
    sink = rng.standard_normal(H)
    return q, v, sel, sink


def test_matches_torch_sdpa_with_sink_as_extra_key():
    q, v, sel, sink = _case(0)
    scale = 0.37
    out = sparse_attention(q, v, sel, sink, scale)
    R, H, D = out.shape
    k = v.shape[1]
    qt = torch.from_numpy(oracle.bf16_bits_to_f64(q))[:, :, None, :]              # [R,H,1,D]
    vt = torch.from_numpy(oracle.bf16_bits_to_f64(v))
    kv = torch.cat([vt, torch.zeros(R, 1, D, dtype=torch.float64)], dim=1)[:, None]  # [R,1,k+1,D]
    mask = torch.zeros(R, H, 1, k + 1, dtype=torch.float64)
    mask[..., :k] = torch.where(torch.from_numpy(sel >= 0)[:, None, None, :], 0.0, float("-inf"))
    mask[..., k] = torch.from_numpy(sink)[None, :, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kv.expand(R, H, k + 1, D), kv.expand(R, H, k + 1, D), attn_mask=mask, scale=scale)
    np.testing.assert_allclose(out, ref[:, :, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_equal_scores_closed_form():
    """q = 0: every valid slot weighs 1 / (n + exp(sink))."""
    _, v, sel, sink = _case(1)
    q = np.zeros((3, 4, 16), np.uint16)
    out = sparse_attention(q, v, sel, sink, 1.0)
    vv = oracle.bf16_bits_to_f64(v)
    for r in range(3):
        ok = sel[r] >= 0
        for h in range(4):
            want = vv[r, ok].sum(axis=0) / (ok.sum() + np.exp(sink[h]))
            np.testing.assert_allclose(out[r, h], want, rtol=1e-13)
    # no sink: the plain mean of the valid rows
    out = sparse_attention(q, v, sel, None, 1.0)
    np.testing.assert_allclose(out[1, 2], vv[1, sel[1] >= 0].mean(axis=0), rtol=1e-13)


def test_limits():
    q, v, sel, sink = _case(2)
    # no valid slot: 0 (all weight on the sink, or nothing at all)
    sel0 = np.full_like(sel, -1)
    assert np.all(sparse_attention(q, v, sel0, sink, 1.0) == 0)
    assert np.all(sparse_attention(q, v, sel0, None, 1.0) == 0)
    # a dominant key takes all the weight; a huge sink takes it away
    D = 16
    v2 = _bf16(np.eye(D)[:9])[None]                     # rows e_0..e_8
    q2 = _bf16(np.eye(D)[[3]] * 4)[None]                # q = 4 e_3: scores 4*scale on slot 3
    s2 = np.zeros((1, 9), np.int32)
    out = sparse_attention(q2, v2, s2, np.array([-50.0]), 20.0)   # score 80 vs 0
    np.testing.assert_allclose(out[0, 0], np.eye(D)[3], atol=1e-30)
    out = sparse_attention(q2, v2, s2, np.array([1e3]), 20.0)
    assert np.abs(out).max() < 1e-300


def test_slot_order_and_padding_do_not_matter():
    q, v, sel, sink = _case(3)
    out = sparse_attention(q, v, sel, sink, 0.5)
    rng = np.random.default_rng(9)
    perm = rng.permutation(v.shape[1])
    np.testing.assert_allclose(sparse_attention(q, v[:, perm], sel[:, perm], sink, 0.5), out, rtol=1e-13)
    # padding slots: whatever their rows hold, nothing changes
    v2 = v.copy()
    v2[sel < 0] = _bf16(np.full(16, 1e4))
    np.testing.assert_allclose(sparse_attention(q, v2, sel, sink, 0.5), out, rtol=0, atol=0)
    # dropping the padding slots of a row leaves that row unchanged
    ok = sel[1] >= 0
    sub = sparse_attention(q[1:2], v[1:2, ok], sel[1:2, ok], sink, 0.5)
    np.testing.assert_allclose(sub[0], out[1], rtol=1e-13)


def test_composes_with_the_gather_oracle():
    """Rows read through the pinned gather oracle from an mxfp4 cache: the
    attention of a slot list equals the attention over its gathered rows
    (the consumer's input is the gather's output)."""
    rng = np.random.default_rng(4)
    NB, bs, R, k = 4, 16, 2, 12
    kv = rng.integers(0, 256, (NB, bs, 64), dtype=np.uint8)
    sc = rng.integers(124, 131, (NB, bs, 4), dtype=np.uint8)
    table = rng.permutation(NB).astype(np.int32)[None, :]
    sel = rng.integers(-1, NB * bs, (R, k)).astype(np.int32)
    rows = oracle.mxfp4_paged_gather(kv, sc, table, sel, np.zeros(R, np.int32), bs)
    q = _bf16(rng.standard_normal((R, 8, 128)) * 0.05)
    out = sparse_attention(q, rows, sel, rng.standard_normal(8), 0.09)
    assert np.all(np.isfinite(out))
    # each output is a convex combination (weights < 1) of the valid rows
    vv = oracle.bf16_bits_to_f64(rows)
    for r in range(R):
        ok = sel[r] >= 0
        lo, hi = vv[r, ok].min(axis=0), vv[r, ok].max(axis=0)
        assert np.all(out[r] <= np.maximum(hi, 0) + 1e-9) and np.all(out[r] >= np.minimum(lo, 0) - 1e-9)
