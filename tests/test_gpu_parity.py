"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Gates (per config):
  logits  masked entries are exactly -inf; over valid entries
          max|gpu - oracle| / max|oracle| <= 1e-3 (bf16) or 5e-2 (fp8); no NaN.
  top-k   bit-exact against the oracle's selection run on the GPU's own logits
          (tie rule: score descending, then lower j; -1 padding). Jaccard
          against the oracle's selection on the oracle's logits is reported.
  gather  bit-exact against the oracle's gather of the same sel_pos.
Outputs are pre-filled with sentinels so that an element a kernel fails to
write shows up.  Full configs run in the same launch configuration as
bench.py; the largest are checked on sampled rows the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-3, "fp8": 5e-2}
SENT_F32 = float("nan")
SENT_I32 = 0x7EADBEEF
SENT_BF16 = 0x7FC1


@pytest.fixture(scope="module")
def xk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_logits_amd as xk
    return xk


def _sample_rows(cfg, n_sample):
    R = cfg.rows
    if R <= n_sample:
        return np.arange(R)
    rng = np.random.default_rng(1234)
    edge = np.array([0, 1, 7, 8, R // 2, R - 9, R - 8, R - 2, R - 1])
    return np.unique(np.concatenate([edge, rng.choice(R, n_sample - edge.size, replace=False)]))


def run_logits(xk, x, d):
    cfg = x["cfg"]
    out = torch.full((cfg.B, cfg.T, cfg.K), SENT_F32, dtype=torch.float32, device="cuda")
    xk.xk_indexer_logits(d["q"], d["k"], d["w"], d["limit"], d["q_scale"], d["k_scale"], out=out)
    torch.cuda.synchronize()
    return out


def check_logits(x, g_np, rows, label=""):
    """g_np: [B,T,K] GPU logits (host). rows: flat row ids to check against the oracle."""
    cfg = x["cfg"]
    pairs = [(int(r) // cfg.T, int(r) % cfg.T) for r in rows]
    o = oracle.indexer_logits(x["q"], x["k"], x["w"], x["limit"], x["q_scale"], x["k_scale"],
                              cfg.dtype, rows=pairs)
    worst = 0.0
    for b, t in pairs:
        n = max(0, min(int(x["limit"][b, t]) + 1, cfg.K))
        g, ref = g_np[b, t], o[b, t]
        assert not np.isnan(g).any(), f"{label} row {(b, t)} has unwritten/NaN entries"
        assert np.all(g[n:] == -np.inf), f"{label} row {(b, t)}: masked entries not -inf"
        if n:
            assert np.all(np.isfinite(g[:n])), f"{label} row {(b, t)}: non-finite valid entry"
            scale = max(float(np.abs(ref[:n]).max()), 1e-30)
            err = float(np.abs(g[:n].astype(np.float64) - ref[:n]).max()) / scale
            worst = max(worst, err)
    assert worst <= TOL[cfg.dtype], f"{label} max rel err {worst:.3e} > {TOL[cfg.dtype]}"
    return worst


def run_topk(xk, logits, limit_flat, k):
    R = logits.shape[0] * logits.shape[1]
    out = torch.full((R, k), SENT_I32, dtype=torch.int32, device="cuda")
    xk.xk_indexer_topk(logits, k, limit_flat, out=out)
    torch.cuda.synchronize()
    return out


def check_topk(g_idx, g_logits_2d, limit_flat, k, rows, label=""):
    ref = oracle.indexer_topk(g_logits_2d, limit_flat, k, rows=rows)
    for r in rows:
        assert np.array_equal(g_idx[r], ref[r]), f"{label} top-k row {r} differs"


def jaccard(a, b):
    sa, sb = set(a[a >= 0].tolist()), set(b[b >= 0].tolist())
    if not sa and not sb:
        return 1.0
    return len(sa & sb) / len(sa | sb)


def run_gather(xk, d, sel_pos_dev, row_seq=True):
    R, k = sel_pos_dev.shape
    out = torch.full((R, k, 128), SENT_BF16, dtype=torch.int16, device="cuda")
    xk.xk_mxfp4_paged_gather(d["kv_fp4"], d["kv_scale"], d["block_table"], sel_pos_dev,
                             d["row_seq"] if row_seq else None, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def assert_sel_pos_in_range(sel, x):
    """Host check before a gather: every index is -1 or inside its row's sequence."""
    lens = x["seq_len"][x["row_seq"]]
    assert np.all(sel >= -1)
    assert np.all(sel < lens[:, None]), "sel_pos outside its sequence"


# ----------------------------------------------------------------------------- configs
# logits rows checked against the oracle (None: every row); the top-k is
# checked on every row of every config (the oracle's selection on the GPU's
# own logits costs a sort per row)
CONFIG_SAMPLES = {"tiny": None, "flash_decode": None, "flash_prefill": None,
                  "pro_decode": None, "long_fp8_prefill": 128}


@pytest.mark.parametrize("name", list(CONFIG_SAMPLES))
def test_config_chain(xk, name):
    """logits -> top-k -> gather on one config, each stage against the oracle."""
    x = workloads.inputs(name)
    cfg = x["cfg"]
    print(f"[parity] config={name} B={cfg.B} T={cfg.T} K={cfg.K} k={cfg.topk} {cfg.dtype}",
          flush=True)
    d = workloads.to_device(x)
    rows = _sample_rows(cfg, CONFIG_SAMPLES[name]) if CONFIG_SAMPLES[name] else np.arange(cfg.rows)

    g_logits = run_logits(xk, x, d)
    g_np = g_logits.cpu().numpy()
    assert not np.isnan(g_np).any(), "unwritten logits"
    err = check_logits(x, g_np, rows, name)

    lim_flat = x["limit"].reshape(-1)
    g_idx = run_topk(xk, g_logits, d["limit"].reshape(-1), cfg.topk).cpu().numpy()
    assert not np.any(g_idx == SENT_I32)
    L2 = g_np.reshape(cfg.rows, cfg.K)
    check_topk(g_idx, L2, lim_flat, cfg.topk, np.arange(cfg.rows), name)
    # selection against the oracle's own logits (P3-style Jaccard report)
    o_log = oracle.indexer_logits(x["q"], x["k"], x["w"], x["limit"], x["q_scale"], x["k_scale"],
                                  cfg.dtype, rows=[(int(r) // cfg.T, int(r) % cfg.T)
                                                   for r in rows[:64]]).reshape(cfg.rows, cfg.K)
    o_idx = oracle.indexer_topk(o_log, lim_flat, cfg.topk, rows=rows[:64])
    jac = [jaccard(g_idx[r], o_idx[r]) for r in rows[:64]]
    print(f"[parity] {name}: logits rel err {err:.2e}, top-k Jaccard vs oracle-logit "
          f"selection mean {np.mean(jac):.4f} min {np.min(jac):.4f}", flush=True)
    assert np.mean(jac) >= (0.999 if cfg.dtype == "bf16" else 0.95)

    sel = workloads.apply_forced_negatives(g_idx, x["neg_slots"])
    assert_sel_pos_in_range(sel, x)
    sel_dev = torch.from_numpy(sel).cuda()
    g_gat = run_gather(xk, d, sel_dev)
    assert not np.any(g_gat == SENT_BF16), "unwritten gather output"  # decode never yields NaN
    grows = rows if rows.size <= 256 else _sample_rows(cfg, 256)
    o_gat = oracle.mxfp4_paged_gather(x["kv_fp4"], x["kv_scale"], x["block_table"], sel,
                                      x["row_seq"], x["block_size"], rows=grows)
    assert np.array_equal(g_gat[grows], o_gat[grows]), f"{name}: gather differs"
    if name == "tiny":
        assert (sel == -1).sum() >= 3 * cfg.rows


def test_tiny_gather_hits_ff_scales(xk):
    """The 0xFF scale bytes planted in the tiny cache, gathered explicitly."""
    x = workloads.inputs("tiny")
    d = workloads.to_device(x)
    ff = x["ff_positions"]                     # flat index into [NB, bs, 4]
    blk, off = ff // (64 * 4), (ff // 4) % 64
    inv = np.empty(4, dtype=np.int64)
    inv[x["block_table"][0]] = np.arange(4)   # physical -> logical block
    pos = (inv[blk] * 64 + off).astype(np.int32)
    sel = np.full((1, 16), -1, np.int32)
    sel[0, : pos.size] = pos
    sel[0, 8:12] = [0, 63, 64, 255]
    g = run_gather(xk, d, torch.from_numpy(sel).cuda(), row_seq=False)
    o = oracle.mxfp4_paged_gather(x["kv_fp4"], x["kv_scale"], x["block_table"], sel,
                                  np.zeros(1, np.int32), 64)
    assert np.array_equal(g, o)
    zeroed = (g[0, : pos.size] & 0x7FFF) == 0
    assert zeroed.sum() >= 32 * pos.size          # each 0xFF group decodes to signed zeros


# ----------------------------------------------------------------------------- edge cases
@pytest.mark.parametrize("B,T,K,lim_mode", [
    (1, 3, 300, "causal"),        # decode path, ragged K
    (2, 13, 1000, "causal"),      # prefill path, ragged T and K
    (3, 9, 4097, "none"),         # no limit array, K one past a tile
    (1, 17, 64, "mixed"),         # negative and >= K limits
    (2, 1, 129, "mixed"),
])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_logits_edges(xk, B, T, K, lim_mode, dtype):
    print(f"[parity] logits edge B={B} T={T} K={K} {lim_mode} {dtype}", flush=True)
    x = workloads.custom(seed=B * 1000 + T * 10 + K, B=B, T=T, K=K, topk=8, dtype=dtype,
                         causal_offset=max(0, K - T - 5) if lim_mode == "causal" else None)
    if lim_mode == "mixed":
        rng = np.random.default_rng(K)
        x["limit"] = rng.choice([-5, -1, 0, 1, K // 2, K - 1, K, K + 100, 2 ** 31 - 1],
                                size=(B, T)).astype(np.int32)
    d = workloads.to_device(x)
    lim = None if lim_mode == "none" else d["limit"]
    out = torch.full((B, T, K), SENT_F32, dtype=torch.float32, device="cuda")
    xk.xk_indexer_logits(d["q"], d["k"], d["w"], lim, d["q_scale"], d["k_scale"], out=out)
    torch.cuda.synchronize()
    if lim_mode == "none":
        x["limit"] = np.full((B, T), K - 1, np.int32)
    check_logits(x, out.cpu().numpy(), np.arange(B * T), f"edge {B},{T},{K}")


@pytest.mark.parametrize("T", [3, 24])  # decode and prefill kernels (both round through f16)
def test_logits_fp8_extremes(xk, T):
    """fp8 inputs at the edges of the f16 epilogue: e4m3 codes over every
    finite value (scores up to 128 * 448^2, just under the 2^25 the block
    scale maps to 1), scales spread over 2^-8 .. 2^8, head weights spanning
    2^-40 .. 2^10 with both signs (the smallest flush to zero in f16 against
    the largest), one query with all weights zero (its valid logits are
    exactly 0) and one with a single nonzero weight. The contract is 5e-2 of
    max|logit|; the f16 roundings are checked against 1e-2."""
    print(f"[parity] logits fp8 extremes T={T}", flush=True)
    K = 700
    x = workloads.custom(seed=4242 + T, B=1, T=T, K=K, topk=8, dtype="fp8", causal_offset=K - T)
    rng = np.random.default_rng(99 + T)
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)  # every finite e4m3 code
    x["q"] = rng.choice(codes, size=x["q"].shape).astype(np.uint8)
    x["k"] = rng.choice(codes, size=x["k"].shape).astype(np.uint8)
    x["k"][0, : K // 8] = 0x7E                            # +448 rows: the largest scores
    x["q_scale"] = np.exp2(rng.uniform(-8, 8, size=x["q_scale"].shape)).astype(np.float32)
    x["k_scale"] = np.exp2(rng.uniform(-8, 8, size=x["k_scale"].shape)).astype(np.float32)
    w = np.exp2(rng.uniform(-40, 10, size=x["w"].shape)) * rng.choice([-1.0, 1.0], size=x["w"].shape)
    w[0, 0] = 0.0
    w[0, 1] = 0.0
    w[0, 1, 5] = 3.0
    x["w"] = w.astype(np.float32)
    d = workloads.to_device(x)
    g = run_logits(xk, x, d).cpu().numpy()
    err = check_logits(x, g, np.arange(T), f"fp8 extremes T={T}")
    assert err <= 1e-2, f"fp8 extremes: rel err {err:.3e}"
    n0 = int(x["limit"][0, 0]) + 1
    assert np.all(g[0, 0, :n0] == 0.0), "all-zero weights must give exact zeros"


def test_logits_deterministic(xk):
    x = workloads.custom(seed=77, B=1, T=40, K=777, dtype="bf16", causal_offset=700)
    d = workloads.to_device(x)
    a = xk.xk_indexer_logits(d["q"], d["k"], d["w"], d["limit"])
    b = xk.xk_indexer_logits(d["q"], d["k"], d["w"], d["limit"])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def _topk_case(xk, L, lim, k):
    Ld = torch.from_numpy(L).cuda()
    limd = None if lim is None else torch.from_numpy(lim).cuda()
    g = run_topk(xk, Ld.view(L.shape[0], 1, L.shape[1]), limd, k).cpu().numpy()
    ref = oracle.indexer_topk(L, lim, k)
    assert np.array_equal(g, ref)
    return g


@pytest.mark.parametrize("K", [1, 5, 300, 1024, 1025, 4096, 5000, 16384, 16385, 40000, 65536,
                               98304, 150001])
@pytest.mark.parametrize("k", [1, 16, 512, 1024, 2048])
def test_topk_random_rows(xk, K, k):
    print(f"[parity] top-k random K={K} k={k}", flush=True)
    rng = np.random.default_rng(K * 7 + k)
    R = 6
    L = rng.standard_normal((R, K)).astype(np.float32)
    lim = np.array([K - 1, K // 2, k - 1, k, -1, K + 5], np.int32)
    _topk_case(xk, L, lim, k)


@pytest.mark.parametrize("K", [700, 5000, 70000])
def test_topk_heavy_ties_and_signed_zero(xk, K):
    print(f"[parity] top-k ties K={K}", flush=True)
    rng = np.random.default_rng(K)
    R = 5
    L = rng.choice(np.float32([0.0, -0.0, 1.0, 2.0, -1.0]), size=(R, K))
    L[1] = 3.0                                            # all equal
    L[2] = -np.arange(K, dtype=np.float32)                # strictly decreasing
    L[3] = np.arange(K, dtype=np.float32)                 # strictly increasing
    L[4, : K // 2] = -np.inf                              # valid -inf keys
    for k in (1, 16, 512, 2048):
        _topk_case(xk, L, None, k)
        _topk_case(xk, L, np.array([K - 1, 10, K // 3, K - 2, K // 2 + 3], np.int32), k)


@pytest.mark.parametrize("K,k", [(98304, 1024), (98304, 2048), (40000, 512)])
def test_topk_long_rows_paired(xk, K, k):
    """Batches of >= 512 long rows run two 512-thread workgroups per CU with a
    6K-entry candidate list that is shrunk (and the bound raised) when it
    fills. Rows: plain normal, upward trends that fill the list (refresh),
    a steep trend and an increasing row that overflow it (radix path),
    heavy ties, all-equal, half -inf, decreasing; mixed limits."""
    print(f"[parity] top-k long paired K={K} k={k}", flush=True)
    rng = np.random.default_rng(K + k)
    R = 512
    L = rng.standard_normal((R, K)).astype(np.float32)
    ramp = np.arange(K, dtype=np.float32) / K
    for r in range(R):
        kind = r % 8
        if kind == 1:
            L[r] += 0.5 * ramp
        elif kind == 2:
            L[r] += 1.0 * ramp
        elif kind == 3:
            L[r] += 4.0 * ramp
        elif kind == 4:
            L[r] = rng.choice(np.float32([0.0, -0.0, 1.0, 2.0, -1.0]), size=K)
        elif kind == 5:
            L[r] = np.arange(K, dtype=np.float32) if r % 16 == 5 else 3.0
        elif kind == 6:
            L[r, : K // 2] = -np.inf
        elif kind == 7 and r % 16 == 7:
            L[r] = -np.arange(K, dtype=np.float32)
    lim = np.full(R, K - 1, np.int32)
    lim[::5] = rng.integers(0, K, size=len(lim[::5]))
    lim[3::11] = K + 7
    _topk_case(xk, L, lim, k)


def test_topk_deterministic(xk):
    rng = np.random.default_rng(3)
    L = torch.from_numpy(rng.choice(np.float32([0, 1, 2]), size=(64, 9000))).cuda()
    a = run_topk(xk, L.view(64, 1, 9000), None, 1024)
    b = run_topk(xk, L.view(64, 1, 9000), None, 1024)
    assert torch.equal(a, b)


def test_gather_golden_bytes_and_scales(xk):
    """Hand-derived golden bytes (tests/golden) through the GPU decode, plus all
    16 codes x extreme scale bytes."""
    from test_oracle_pins import _golden_rows
    rows = _golden_rows()
    bs = 16
    codes = np.arange(256, dtype=np.uint8)
    scales = np.array([0, 1, 2, 118, 120, 127, 128, 134, 136, 252, 253, 254, 255], np.uint8)
    NB = 1 + len(scales) * 256 // bs
    fp4 = np.zeros((NB, bs, 64), np.uint8)
    sc = np.full((NB, bs, 4), 127, np.uint8)
    for i, (p, s, _, _) in enumerate(rows):
        fp4[0, i, :] = p
        sc[0, i, :] = s
    tok = bs
    for s in scales:
        for c in codes:
            fp4.reshape(-1, 64)[tok] = c
            sc.reshape(-1, 4)[tok] = s
            tok += 1
    n_tok = tok
    table = np.arange(NB, dtype=np.int32)[None]
    sel = np.full((1, ((n_tok + 15) // 16) * 16), -1, np.int32)
    sel[0, :n_tok] = np.arange(n_tok)
    d = {"kv_fp4": torch.from_numpy(fp4).cuda(), "kv_scale": torch.from_numpy(sc).cuda(),
         "block_table": torch.from_numpy(table).cuda(), "row_seq": torch.zeros(1, dtype=torch.int32).cuda()}
    g = run_gather(xk, d, torch.from_numpy(sel).cuda())
    for i, (_, _, lo, hi) in enumerate(rows):
        assert np.all(g[0, i, 0::2] == lo) and np.all(g[0, i, 1::2] == hi), i
    o = oracle.mxfp4_paged_gather(fp4, sc, table, sel, np.zeros(1, np.int32), bs)
    assert np.array_equal(g, o)


# k = 33: workgroups take consecutive slots; k = 64, 96: rows of whole workgroups, grouped by
# XCD, with 5 rows (not a multiple of 8)
@pytest.mark.parametrize("k", [33, 64, 96])
@pytest.mark.parametrize("bs", [1, 16, 64, 256])
def test_gather_block_sizes_and_identity_rows(xk, bs, k):
    print(f"[parity] gather bs={bs} k={k}", flush=True)
    rng = np.random.default_rng(bs * 1000 + k)
    S, MB = 5, 7
    NB = S * MB
    fp4 = rng.integers(0, 256, size=(NB, bs, 64), dtype=np.uint8)
    sc = rng.integers(110, 145, size=(NB, bs, 4), dtype=np.uint8)
    sc[rng.random(sc.shape) < 0.05] = 0xFF
    table = rng.permutation(NB).astype(np.int32).reshape(S, MB)
    R = S
    sel = rng.integers(-2, MB * bs, size=(R, k)).astype(np.int32)
    d = {"kv_fp4": torch.from_numpy(fp4).cuda(), "kv_scale": torch.from_numpy(sc).cuda(),
         "block_table": torch.from_numpy(table).cuda(), "row_seq": None}
    g = run_gather(xk, d, torch.from_numpy(sel).cuda(), row_seq=False)
    o = oracle.mxfp4_paged_gather(fp4, sc, table, sel, np.arange(R, dtype=np.int32), bs)
    assert np.array_equal(g, o)
    assert np.all(g[sel < 0] == 0)
