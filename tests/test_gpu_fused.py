"""Parity of xk_indexer_logits_topk (fused logits -> top-k) through the C ABI.

The fused call is defined as the composition xk_indexer_topk(xk_indexer_logits
(...)), so its output must equal, element for element:
  * the oracle's selection (oracle.indexer_topk, pinned on its own) from the
    GPU's scores, on sampled rows, and
  * the unfused GPU chain on the same inputs, on every row.
The scores themselves are checked against the oracle's float64 scores by the
logits parity tests. Cases cover the candidate path (long and short causal
rows, ragged query blocks, several sequences, no limit, negative and clamped
limits, k from 16 to 2048), the recompute path (candidate regions that
overflow: scores rising with j, and exact ties on every key), the branch
through the score matrix (few queries, few keys per index), both prefill
configs and HIP-graph replay.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

SENTINEL = 0x7EADBEEF


@pytest.fixture(scope="module")
def xk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_logits_amd as xk
    return xk


def _fused_plan(xk, B, T, K, k, fp8):
    """True when the call takes the candidate path (its workspace is not the
    score matrix)."""
    ws = xk.xk_indexer_logits_topk_workspace_size(B, T, K, k, 1 if fp8 else 0)
    return ws != (B * T * K * 4 + 255) // 256 * 256


def _run(xk, d, k, limit):
    lg = xk.xk_indexer_logits(d["q"], d["k"], d["w"], limit, d["q_scale"], d["k_scale"])
    R = lg.shape[0] * lg.shape[1]
    ref = xk.xk_indexer_topk(lg, k, None if limit is None else limit.reshape(-1))
    got = torch.full((R, k), SENTINEL, dtype=torch.int32, device="cuda")
    xk.xk_indexer_logits_topk(d["q"], d["k"], d["w"], k, limit, d["q_scale"], d["k_scale"], out=got)
    torch.cuda.synchronize()
    return lg, ref, got


def _check(xk, d, k, limit, label, n_sample=12, seed=0):
    lg, ref, got = _run(xk, d, k, limit)
    B, T, K = lg.shape
    R = B * T
    g = got.cpu().numpy()
    assert not (g == SENTINEL).any(), f"{label}: unwritten output"
    rows = np.unique(np.r_[0, R - 1, np.random.default_rng(seed).choice(R, n_sample)])
    lim = None if limit is None else limit.reshape(-1).cpu().numpy()
    o = oracle.indexer_topk(lg.reshape(R, K).cpu().numpy(), lim, k, rows=rows)
    for r in rows:
        assert np.array_equal(g[r], o[r]), f"{label}: row {r} differs from the oracle's selection"
    assert torch.equal(got, ref), f"{label}: differs from the unfused chain"
    return g


@pytest.mark.parametrize("B,T,K,k,dtype,causal_offset,len_range", [
    (1, 2048, 20000, 1024, "fp8", 17952, None),   # long causal rows
    (1, 2048, 16384, 1024, "fp8", 0, None),       # short causal rows: fewer than k keys, -1 padding
    (1, 1021, 9000, 512, "bf16", 8000, None),     # ragged last query block
    (2, 512, 6000, 256, "bf16", None, (1000, 6000)),  # two sequences, per-sequence lengths
    (1, 2048, 40000, 2048, "fp8", 37952, None),   # the largest k (64 x 32-entry lane lists)
    (1, 2048, 5000, 16, "fp8", 2952, None),       # a small k
])
def test_fused_matches_composition(xk, B, T, K, k, dtype, causal_offset, len_range):
    x = workloads.custom(seed=B * 7 + T + K, B=B, T=T, K=K, topk=k, dtype=dtype,
                         causal_offset=causal_offset, len_range=len_range)
    assert _fused_plan(xk, B, T, K, k, dtype == "fp8")
    print(f"[fused] B={B} T={T} K={K} k={k} {dtype}", flush=True)
    d = workloads.to_device(x)
    _check(xk, d, k, d["limit"], f"B={B} T={T} K={K} k={k}")


def test_fused_limits(xk):
    """No limit at all; then negative limits (empty rows), limits past K and
    single-key rows."""
    B, T, K, k = 1, 2048, 20000, 512
    x = workloads.custom(seed=11, B=B, T=T, K=K, topk=k, dtype="fp8", causal_offset=K - T)
    d = workloads.to_device(x)
    _check(xk, d, k, None, "no limit")
    lim = x["limit"].copy()
    lim[0, 3::11] = K + 100
    lim[0, 5::13] = 0
    lim[0, ::7] = -1
    d["limit"] = torch.from_numpy(lim).cuda()
    g = _check(xk, d, k, d["limit"], "edge limits")
    assert np.all(g[::7] == -1)


def _monotone_fp8(T, K, k, tie):
    """Scores that rise with j (or are all equal): every key beats the bound
    seen so far, so the candidate regions overflow and every row is
    recomputed. q and k bytes are all e4m3 1.0, w > 0; the per-key scale
    orders the scores."""
    x = workloads.custom(seed=21, B=1, T=T, K=K, topk=k, dtype="fp8", causal_offset=K - T)
    x = dict(x)
    x["q"] = np.full_like(x["q"], 0x38)
    x["k"] = np.full_like(x["k"], 0x38)
    x["w"] = (np.abs(x["w"]) + 0.01).astype(np.float32)
    x["k_scale"] = (np.full(x["k_scale"].shape, 0.01, np.float32) if tie else
                    np.linspace(0.01, 1.0, K, dtype=np.float32)[None, :])
    return x


@pytest.mark.parametrize("tie", [False, True])
def test_fused_recompute_path_fp8(xk, tie):
    T, K, k = 2048, 20000, 1024
    x = _monotone_fp8(T, K, k, tie)
    print(f"[fused] recompute fp8 tie={tie}", flush=True)
    d = workloads.to_device(x)
    g = _check(xk, d, k, d["limit"], f"recompute tie={tie}")
    if tie:   # all scores equal: the lowest j win, in order
        assert np.array_equal(g[0], np.arange(k))
    else:     # rising scores: the last k valid keys, highest first
        n = int(x["limit"][0, 0]) + 1
        assert np.array_equal(g[0], np.arange(n - 1, n - 1 - k, -1))


def test_fused_recompute_path_bf16(xk):
    """bf16 keys v_j = bf16(0.5 + j/K) on every dimension: non-decreasing
    scores with runs of exact ties."""
    T, K, k = 1024, 20000, 512
    x = dict(workloads.custom(seed=23, B=1, T=T, K=K, topk=k, dtype="bf16", causal_offset=K - T))
    one = np.uint16(0x3F80)
    x["q"] = np.full_like(x["q"], one)
    v = torch.from_numpy((0.5 + np.arange(K) / K).astype(np.float32)).to(torch.bfloat16)
    x["k"] = np.repeat(v.view(torch.int16).numpy().view(np.uint16)[None, :, None], 128, axis=2)
    x["w"] = (np.abs(x["w"]) + 0.01).astype(np.float32)
    d = workloads.to_device(x)
    _check(xk, d, k, d["limit"], "recompute bf16")


def test_fused_few_queries_branch(xk):
    """Decode shapes: the scores go through the workspace, same results."""
    x = workloads.custom(seed=31, B=4, T=1, K=3000, topk=512, dtype="bf16", len_range=(100, 3000))
    assert not _fused_plan(xk, 4, 1, 3000, 512, False)
    d = workloads.to_device(x)
    _check(xk, d, 512, d["limit"], "few queries")


@pytest.mark.parametrize("name", ["flash_prefill", "long_fp8_prefill"])
def test_fused_config(xk, name):
    """The long-context config takes the candidate path; the Flash prefill
    config (8 keys per selected index) goes through the score matrix."""
    x = workloads.inputs(name)
    cfg = x["cfg"]
    assert _fused_plan(xk, cfg.B, cfg.T, cfg.K, cfg.topk, cfg.dtype == "fp8") == (name == "long_fp8_prefill")
    print(f"[fused] config={name}", flush=True)
    d = workloads.to_device(x)
    _check(xk, d, cfg.topk, d["limit"], name, n_sample=6)


def test_fused_graph_replays(xk):
    """Captured in a HIP graph (the workspace counters are cleared by a kernel,
    not a memset), replays match eager, with eager work between replays."""
    x = workloads.custom(seed=41, B=1, T=2048, K=17000, topk=1024, dtype="fp8", causal_offset=14952)
    assert _fused_plan(xk, 1, 2048, 17000, 1024, True)
    d = workloads.to_device(x)
    _, out, ws = xk.logits_topk_args(d["q"], d["k"], d["w"], 1024, d["limit"], d["q_scale"],
                                     d["k_scale"])

    def call():
        xk.xk_indexer_logits_topk(d["q"], d["k"], d["w"], 1024, d["limit"], d["q_scale"],
                                  d["k_scale"], out=out, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        out.fill_(-7)
        ws.fill_(0xA5)        # stale workspace contents must not matter
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from eager"
        xk.xk_indexer_logits_topk(d["q"], d["k"], d["w"], 64, d["limit"], d["q_scale"], d["k_scale"])
        torch.cuda.synchronize()
