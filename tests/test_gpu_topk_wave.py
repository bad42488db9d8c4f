"""Parity of the top-k's one-wave-per-row path (many rows of at most 4096
keys, k <= 512, K a multiple of 4) with the oracle, through the C ABI.

The batches have at least 1024 rows, so the launcher takes that path; each
mixes rows the wave finishes itself with rows it hands to the workgroup's
radix path (more than 896 candidates above the bound, the wave's list size:
heavy ties, infinities), and the row count is not a multiple of the rows per
workgroup. Every row is compared with the oracle, bit for bit."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

SENT = np.int32(-0x5A5A5A5A)


@pytest.fixture(scope="module")
def xk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_logits_amd as xk
    return xk


def _check(xk, L, lim, k, label):
    R, K = L.shape
    out = torch.full((R, k), int(SENT), dtype=torch.int32, device="cuda")
    Ld = torch.from_numpy(L).cuda()
    xk.xk_indexer_topk(Ld.view(R, 1, K), k, None if lim is None else torch.from_numpy(lim).cuda(), out=out)
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    ref = oracle.indexer_topk(L, lim, k)
    bad = np.nonzero((g != ref).any(axis=1))[0]
    assert bad.size == 0, f"{label}: {bad.size} rows differ, first {bad[:8].tolist()}"


def _limits(rng, R, K, k):
    """Causal rows (limit = row index mod K) plus the edges: empty rows,
    fewer valid keys than k, exactly k, past the end, random."""
    lim = (np.arange(R) % K).astype(np.int32)
    lim[rng.choice(R, 12, replace=False)] = -1
    lim[rng.choice(R, 8, replace=False)] = k - 2
    lim[rng.choice(R, 8, replace=False)] = k - 1
    lim[rng.choice(R, 8, replace=False)] = K + 9
    sel = rng.choice(R, R // 4, replace=False)
    lim[sel] = rng.integers(-1, K, sel.size)
    return lim


@pytest.mark.parametrize("K", [64, 1000, 1024, 2048, 2052, 4096])
@pytest.mark.parametrize("k", [1, 16, 512])
def test_wave_topk_random_rows(xk, K, k):
    print(f"[topk-wave] random K={K} k={k}", flush=True)
    rng = np.random.default_rng(K * 31 + k)
    R = 1027
    L = rng.standard_normal((R, K)).astype(np.float32)
    L[5] *= 1e-30                          # a tiny range
    L[6] = L[6] * 1e30                     # a huge range
    _check(xk, L, _limits(rng, R, K, k), k, f"K={K} k={k}")
    _check(xk, L, None, k, f"K={K} k={k} no limit")


@pytest.mark.parametrize("K", [1024, 4096])
def test_wave_topk_ties_infinities_and_fallback(xk, K):
    """Rows the wave orders with crowded bins (few distinct values, short
    rows) and rows it hands back (all equal, long rows of three values,
    infinities stretching the range), in one batch."""
    print(f"[topk-wave] ties K={K}", flush=True)
    rng = np.random.default_rng(K + 5)
    R = 1030
    L = rng.standard_normal((R, K)).astype(np.float32)
    L[0::7] = rng.choice(np.float32([0.0, -0.0, 1.0, 2.0]), size=L[0::7].shape)
    L[1::7] = 3.0
    L[2::7, ::5] = np.inf
    L[3::7, 1::3] = -np.inf
    L[4::7] = -np.arange(K, dtype=np.float32)
    L[5::7] = np.arange(K, dtype=np.float32)
    L[6::14, :] = np.float32(1e38) * rng.choice(np.float32([-3.0, 3.0]), size=L[6::14].shape)  # overflowing range
    for k in (16, 512):
        _check(xk, L, _limits(rng, R, K, k), k, f"ties K={K} k={k}")


def test_wave_topk_deterministic(xk):
    rng = np.random.default_rng(11)
    R, K = 2048, 4096
    L = torch.from_numpy(rng.choice(np.float32([0, 1, 2, 3, 4, 5, 6, 7]), size=(R, K))).cuda()
    L[::2] = torch.from_numpy(rng.standard_normal((R // 2, K)).astype(np.float32)).cuda()
    a = torch.empty((R, 512), dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    xk.xk_indexer_topk(L.view(R, 1, K), 512, None, out=a)
    xk.xk_indexer_topk(L.view(R, 1, K), 512, None, out=b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
