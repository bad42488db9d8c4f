"""Parity of xk_sparse_attention_mxfp4 (the consumer of the selection) with the
oracle, through the C ABI.

The oracle composes the pinned gather oracle (the rows of the selected
positions, decoded exactly) with oracle.sparse_attention (float64). The kernel
decodes the same rows exactly, scores and sums in fp32, and enters the
weights into the value sum rounded to bf16 (relative error at most 2^-8, the
unit roundoff) while the denominator sums them in fp32, so per row
|gpu - oracle| <= 2^-8 * max_j |v_j| up to fp32 rounding. The gate is that
bound (2^-8 of max|v| over the row's valid slots); measured errors are about
1e-3 of max|v|, since the largest weight is exactly 1. A row without a valid
slot is exactly 0.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = 2.0 ** -8


@pytest.fixture(scope="module")
def xk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_logits_amd as xk
    return xk


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def check(xk, q, kv, ks, table, sel, row_seq, sink, scale, bs, label):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    xk.xk_sparse_attention_mxfp4(dev(q.view(np.int16)).view(torch.bfloat16), dev(kv), dev(ks), dev(table), dev(sel),
                                 None if row_seq is None else dev(row_seq),
                                 None if sink is None else dev(np.asarray(sink, np.float32)), scale, out=out)
    torch.cuda.synchronize()
    g = out.cpu().numpy().astype(np.float64)
    rs = np.arange(sel.shape[0], dtype=np.int32) if row_seq is None else row_seq
    rows = oracle.mxfp4_paged_gather(kv, ks, table, sel, rs, bs)
    ref = oracle.sparse_attention(q, rows, sel, sink, scale)
    v = oracle.bf16_bits_to_f64(rows)
    worst = 0.0
    for r in range(sel.shape[0]):
        ok = sel[r] >= 0
        assert np.all(np.isfinite(g[r])), f"{label} row {r}: non-finite output"
        if not ok.any():
            assert np.all(g[r] == 0), f"{label} row {r}: no valid slot but nonzero output"
            continue
        vmax = np.abs(v[r, ok]).max()
        err = np.abs(g[r] - ref[r]).max() / max(vmax, 1e-300)
        worst = max(worst, err)
    assert worst <= TOL, f"{label}: max err {worst:.3e} of max|v|"
    return g, worst


def _cache(rng, NB, bs, lo=124, hi=130, n_ff=0):
    kv = rng.integers(0, 256, (NB, bs, 64), dtype=np.uint8)
    ks = rng.integers(lo, hi + 1, (NB, bs, 4), dtype=np.uint8)
    if n_ff:
        ks.reshape(-1)[rng.choice(ks.size, n_ff, replace=False)] = 0xFF
    return kv, ks


@pytest.mark.parametrize("R,H,k,bs,with_sink", [
    (3, 64, 1, 16, True),        # one slot
    (5, 64, 50, 16, True),       # less than a chunk
    (4, 64, 64, 64, False),      # exactly one chunk, no sink
    (6, 128, 100, 64, True),     # two head groups, ragged last chunk
    (3, 64, 1000, 64, True),     # many chunks
    (2, 64, 2048, 16, True),     # the largest k
])
def test_attention_small(xk, R, H, k, bs, with_sink):
    rng = np.random.default_rng(R * 1000 + k)
    S, MB = 3, 40
    NB = S * MB
    kv, ks = _cache(rng, NB, bs, n_ff=5)
    table = rng.permutation(NB).astype(np.int32).reshape(S, MB)
    sel = rng.integers(0, MB * bs, (R, k)).astype(np.int32)
    sel[rng.random((R, k)) < 0.1] = -1                       # padded slots
    if R > 3:
        sel[3] = -1                                          # a row with no valid slot
    row_seq = rng.integers(0, S, R).astype(np.int32)
    q = _bf16(rng.standard_normal((R, H, 128)) * 0.3)
    sink = rng.standard_normal(H) if with_sink else None
    print(f"[attn] R={R} H={H} k={k} bs={bs} sink={with_sink}", flush=True)
    _, err = check(xk, q, kv, ks, table, sel, row_seq, sink, 0.09, bs, f"R={R} k={k}")
    print(f"[attn] max err {err:.2e}", flush=True)


def test_attention_rows_kernel_at_the_largest_k(xk):
    """Enough rows for the per-row kernel (R*H/64 >= 256 workgroups) at
    k = 2048, the most slots a row may select, with padded slots, a row with
    none, a ragged tail of valid slots and 0xFF scale bytes; sampled rows
    against the oracle."""
    rng = np.random.default_rng(2048)
    R, H, k, bs = 300, 64, 2048, 64
    S, MB = 4, 48
    NB = S * MB
    kv, ks = _cache(rng, NB, bs, n_ff=9)
    table = rng.permutation(NB).astype(np.int32).reshape(S, MB)
    sel = rng.integers(0, MB * bs, (R, k)).astype(np.int32)
    sel[rng.random((R, k)) < 0.05] = -1
    sel[7] = -1                                   # a row with no valid slot
    sel[11, 1500:] = -1                           # valid slots end inside a chunk
    row_seq = rng.integers(0, S, R).astype(np.int32)
    q = _bf16(rng.standard_normal((R, H, 128)) * 0.3)
    sink = rng.standard_normal(H)
    rows = np.unique(np.r_[0, 7, 11, R - 1, rng.choice(R, 12)])
    print(f"[attn] rows kernel R={R} k={k}", flush=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    xk.xk_sparse_attention_mxfp4(dev(q.view(np.int16)).view(torch.bfloat16), dev(kv), dev(ks), dev(table),
                                 dev(sel), dev(row_seq), dev(np.asarray(sink, np.float32)), 0.09, out=out)
    torch.cuda.synchronize()
    g = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), "unwritten or non-finite output"
    gathered = oracle.mxfp4_paged_gather(kv, ks, table, sel[rows], row_seq[rows], bs)
    ref = oracle.sparse_attention(q[rows], gathered, sel[rows], sink, 0.09)
    v = oracle.bf16_bits_to_f64(gathered)
    for i, r in enumerate(rows):
        ok = sel[r] >= 0
        if not ok.any():
            assert np.all(g[r] == 0), f"row {r}: no valid slot but nonzero output"
            continue
        err = np.abs(g[r] - ref[i]).max() / np.abs(v[i, ok]).max()
        assert err <= TOL, f"row {r}: err {err:.3e}"


@pytest.mark.parametrize("regime", ["flat", "peaked", "sink_dominant"])
def test_attention_regimes(xk, regime):
    """Nearly uniform weights, one dominant key, and a sink that takes almost
    all the weight."""
    rng = np.random.default_rng(7)
    R, H, k, bs, NB = 4, 64, 300, 64, 64
    kv, ks = _cache(rng, NB, bs)
    table = np.arange(NB, dtype=np.int32)[None, :]
    sel = rng.integers(0, NB * bs, (R, k)).astype(np.int32)
    sig, sink = {"flat": (1e-3, rng.standard_normal(H)), "peaked": (3.0, rng.standard_normal(H)),
                 "sink_dominant": (0.1, np.full(H, 40.0))}[regime]
    q = _bf16(rng.standard_normal((R, H, 128)) * sig)
    check(xk, q, kv, ks, table, sel, np.zeros(R, np.int32), sink, 0.09, bs, regime)


@pytest.mark.parametrize("name", ["tiny", "flash_decode", "flash_prefill", "long_fp8_prefill"])
def test_attention_config_chain(xk, name):
    """The consumer on a config's GPU selection (top-k of the GPU logits) and
    its mxfp4 cache: sampled rows against the oracle, and a second call
    bit-identical to the first."""
    x = workloads.inputs(name)
    cfg = x["cfg"]
    a = workloads.attention_inputs(cfg)
    print(f"[attn] config={name}", flush=True)
    d = workloads.to_device(x)
    lg = xk.xk_indexer_logits(d["q"], d["k"], d["w"], d["limit"], d["q_scale"], d["k_scale"])
    idx = xk.xk_indexer_topk(lg, cfg.topk, d["limit"].reshape(-1))
    del lg
    q = torch.from_numpy(a["q"].view(np.int16)).cuda().view(torch.bfloat16)
    sink = torch.from_numpy(a["sink"]).cuda()
    o1 = xk.xk_sparse_attention_mxfp4(q, d["kv_fp4"], d["kv_scale"], d["block_table"], idx, d["row_seq"], sink,
                                      a["scale"])
    o2 = xk.xk_sparse_attention_mxfp4(q, d["kv_fp4"], d["kv_scale"], d["block_table"], idx, d["row_seq"], sink,
                                      a["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "not deterministic"
    rows = np.unique(np.r_[0, cfg.rows - 1, np.random.default_rng(1).choice(cfg.rows, min(cfg.rows, 62))])
    sel = idx.cpu().numpy()[rows]
    g = o1.cpu().numpy()[rows].astype(np.float64)
    gathered = oracle.mxfp4_paged_gather(x["kv_fp4"], x["kv_scale"], x["block_table"], sel,
                                         x["row_seq"][rows], x["block_size"])
    ref = oracle.sparse_attention(a["q"][rows], gathered, sel, a["sink"], a["scale"])
    v = oracle.bf16_bits_to_f64(gathered)
    for i, r in enumerate(rows):
        ok = sel[i] >= 0
        vmax = np.abs(v[i, ok]).max() if ok.any() else 1.0
        err = np.abs(g[i] - ref[i]).max() / vmax
        assert err <= TOL, f"{name} row {r}: err {err:.3e}"
