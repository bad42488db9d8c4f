"""Parity of xk_indexer_logits_paged (keys in a paged mxfp4 / fp8 cache)
against the oracle, through the C ABI, and of the whole chain on the paged
bench configs.

The kernel multiplies exact fp8 x E2M1 (or fp8 x fp8) products with exact
power-of-two block scales and accumulates in fp32, so the gate is the dense
bf16 one: max|gpu - oracle| / max|oracle| <= 1e-3 over valid entries,
masked entries exactly -inf, no NaN.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module")
def xk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_logits_amd as xk
    return xk


def run_paged(xk, x, d):
    cfg = x["cfg"]
    out = torch.full((cfg.B, cfg.T, cfg.K), float("nan"), dtype=torch.float32, device="cuda")
    xk.xk_indexer_logits_paged(d["q"], d["q_scale"], d["w"], d["kc"], d["kc_scale"],
                               d["block_table"], d["limit"], K=cfg.K, out=out)
    torch.cuda.synchronize()
    return out


def check(x, g, rows, label):
    cfg = x["cfg"]
    pairs = [(int(r) // cfg.T, int(r) % cfg.T) for r in rows]
    o = oracle.indexer_logits_paged(x["q"], x["q_scale"], x["w"], x["limit"], x["kc"],
                                    x["kc_scale"], x["block_table"], x["block_size"], cfg.K,
                                    cfg.kcache, rows=pairs)
    worst = 0.0
    for b, t in pairs:
        n = max(0, min(int(x["limit"][b, t]) + 1, cfg.K))
        gr, orow = g[b, t], o[b, t]
        assert not np.isnan(gr).any(), f"{label} row {(b, t)}: unwritten entries"
        assert np.all(gr[n:] == -np.inf), f"{label} row {(b, t)}: masked entries not -inf"
        if n:
            assert np.all(np.isfinite(gr[:n])), f"{label} row {(b, t)}: non-finite entry"
            scale = max(float(np.abs(orow[:n]).max()), 1e-30)
            worst = max(worst, float(np.abs(gr[:n].astype(np.float64) - orow[:n]).max()) / scale)
    assert worst <= TOL, f"{label}: max rel err {worst:.3e}"
    return worst


def _paged_case(kcache, B, T, K, lens, seed, n_ff=0, kscale=(120, 134)):
    return workloads.custom(name=f"paged_{kcache}", seed=seed, B=B, T=T, K=K, topk=16,
                            dtype="fp8", len_range=lens, n_ff=n_ff, kcache=kcache,
                            kscale_lo=kscale[0], kscale_hi=kscale[1])


@pytest.mark.parametrize("kcache", ["mxfp4", "fp8"])
@pytest.mark.parametrize("B,T,K,lens", [
    (1, 1, 64, (64, 64)),          # one 64-position page
    (3, 2, 700, (1, 700)),         # ragged lengths, down to a single key
    (2, 5, 1500, (900, 1500)),     # several chunks per row, partial last page
])
def test_paged_logits_small(xk, kcache, B, T, K, lens):
    x = _paged_case(kcache, B, T, K, lens, seed=B * 100 + K, n_ff=6 if kcache == "mxfp4" else 0)
    print(f"[paged] {kcache} B={B} T={T} K={K} lens={lens}", flush=True)
    d = workloads.to_device(x)
    g = run_paged(xk, x, d).cpu().numpy()
    err = check(x, g, np.arange(x["cfg"].rows), kcache)
    print(f"[paged] {kcache}: max rel err {err:.2e}", flush=True)


@pytest.mark.parametrize("bs", [16, 256])
def test_paged_logits_block_sizes(xk, bs):
    """Other page sizes: the cache rebuilt with bs-position pages (same keys)."""
    x = _paged_case("mxfp4", 2, 3, 1000, (300, 1000), seed=7, n_ff=4)
    cfg = x["cfg"]
    lens = x["seq_len"]
    MB = (cfg.K + bs - 1) // bs
    nblk = (lens + bs - 1) // bs
    NB = int(nblk.sum()) + 1
    rng = np.random.default_rng(bs)
    perm = rng.permutation(NB).astype(np.int32)
    table = np.zeros((cfg.B, MB), dtype=np.int32)
    kc = np.zeros((NB, bs, 64), dtype=np.uint8)
    ks = np.full((NB, bs, 4), 127, dtype=np.uint8)
    off = 0
    for b in range(cfg.B):
        table[b, : nblk[b]] = perm[off: off + nblk[b]]
        off += int(nblk[b])
        p = np.arange(int(lens[b]))
        src_blk = x["block_table"][b, p // 64]
        kc[table[b, p // bs], p % bs] = x["kc"][src_blk, p % 64]
        ks[table[b, p // bs], p % bs] = x["kc_scale"][src_blk, p % 64]
    y = dict(x, kc=kc, kc_scale=ks, block_table=table, block_size=bs)
    d = workloads.to_device(y)
    d["kc"], d["kc_scale"] = torch.from_numpy(kc).cuda(), torch.from_numpy(ks).cuda()
    d["block_table"] = torch.from_numpy(table).cuda()
    g = run_paged(xk, y, d).cpu().numpy()
    check(y, g, np.arange(cfg.rows), f"bs={bs}")
    # and the same logits as with 64-position pages
    d64 = workloads.to_device(x)
    g64 = run_paged(xk, x, d64).cpu().numpy()
    assert np.array_equal(g, g64)


def test_paged_logits_limits(xk):
    """Causal limits inside pages, a negative limit and a limit past K."""
    x = _paged_case("mxfp4", 2, 4, 900, (900, 900), seed=31)
    x = dict(x, limit=np.array([[899, 500, -1, 16], [0, 15, 63, 64]], dtype=np.int32))
    d = workloads.to_device(x)
    d["limit"] = torch.from_numpy(x["limit"]).cuda()
    g = run_paged(xk, x, d).cpu().numpy()
    check(x, g, np.arange(8), "limits")


@pytest.mark.parametrize("name", ["flash_decode_fp4", "pro_decode_fp4"])
def test_paged_config_chain(xk, name):
    """The bench configs: paged logits (sampled rows), top-k on the GPU's
    logits and the gather, bit-exact on every row."""
    x = workloads.inputs(name)
    cfg = x["cfg"]
    print(f"[paged] config={name}", flush=True)
    d = workloads.to_device(x)
    g_t = run_paged(xk, x, d)
    g = g_t.cpu().numpy()
    rows = np.unique(np.r_[0, cfg.rows - 1, np.random.default_rng(0).choice(cfg.rows, 12)])
    err = check(x, g, rows, name)
    idx = torch.full((cfg.rows, cfg.topk), 0x7EADBEEF, dtype=torch.int32, device="cuda")
    xk.xk_indexer_topk(g_t, cfg.topk, d["limit"].reshape(-1), out=idx)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    ref = oracle.indexer_topk(g.reshape(cfg.rows, cfg.K), x["limit"].reshape(-1), cfg.topk)
    assert np.array_equal(gi, ref)
    lens = x["seq_len"][x["row_seq"]]
    assert np.all(gi >= -1) and np.all(gi < lens[:, None])
    out = torch.full((cfg.rows, cfg.topk, 128), 0x7FC1, dtype=torch.int16, device="cuda")
    xk.xk_mxfp4_paged_gather(d["kv_fp4"], d["kv_scale"], d["block_table"], idx, d["row_seq"], out=out)
    torch.cuda.synchronize()
    go = out.cpu().numpy().view(np.uint16)
    o = oracle.mxfp4_paged_gather(x["kv_fp4"], x["kv_scale"], x["block_table"], gi, x["row_seq"],
                                  x["block_size"])
    assert np.array_equal(go, o)
    print(f"[paged] {name}: logits rel err {err:.2e}", flush=True)
