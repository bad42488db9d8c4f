"""xk_indexer_logits_topk_noalloc (the fused logits -> top-k entry point
that allocates nothing) through the C ABI, against xk_indexer_logits_topk.

The no-allocation call must write exactly what the workspace call writes
for the same arguments, element for element. Calls run back to back on one
stream, so the built-in scratch holds the previous call's contents when the
next starts: first the long fp8 prefill config (its workspace, ~280 MiB, is
more than the 64 MiB scratch, so the call is split into query ranges), then
a smaller bf16 prefill (one slice), then a decode batch.
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

SENTINEL = 0x7EADBEEF


@pytest.fixture(scope="module")
def xk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_logits_amd as xk
    return xk


def _noalloc(xk, d, k, limit):
    """The C entry point called directly (ctypes), output pre-filled with a sentinel."""
    q, kk, w = d["q"], d["k"], d["w"]
    B, T, H, D = q.shape
    K = kk.shape[1]
    out = torch.full((B * T, k), SENTINEL, dtype=torch.int32, device="cuda")
    dtype = xk.XK_BF16 if q.dtype == torch.bfloat16 else xk.XK_FP8_E4M3_OCP
    st = xk.lib().xk_indexer_logits_topk_noalloc(
        q.data_ptr(), xk._ptr(d["q_scale"]), kk.data_ptr(), xk._ptr(d["k_scale"]), w.data_ptr(),
        xk._ptr(limit), out.data_ptr(), B, T, K, H, D, k, dtype, xk._stream(None))
    assert st == xk.XK_OK, xk.lib().xk_last_error().decode()
    return out


def _check(xk, d, k, limit, label):
    got = _noalloc(xk, d, k, limit)
    ref = xk.xk_indexer_logits_topk(d["q"], d["k"], d["w"], k, limit, d["q_scale"], d["k_scale"])
    torch.cuda.synchronize()
    g, r = got.cpu().numpy(), ref.cpu().numpy()
    assert not (g == SENTINEL).any(), f"{label}: unwritten output"
    bad = np.nonzero((g != r).any(axis=1))[0]
    assert bad.size == 0, f"{label}: rows {bad[:8]} differ from xk_indexer_logits_topk"


def test_noalloc_two_calls_second_smaller(xk):
    x = workloads.inputs("long_fp8_prefill")
    cfg = x["cfg"]
    assert xk.xk_indexer_logits_topk_workspace_size(cfg.B, cfg.T, cfg.K, cfg.topk, 1) > 64 << 20
    print(f"[no-alloc] {cfg.name} B={cfg.B} T={cfg.T} K={cfg.K} k={cfg.topk} (split)", flush=True)
    d = workloads.to_device(x)
    _check(xk, d, cfg.topk, d["limit"], cfg.name)
    del d
    y = workloads.custom(seed=77, B=2, T=40, K=3000, topk=64, dtype="bf16", causal_offset=2900)
    print("[no-alloc] bf16 B=2 T=40 K=3000 k=64 (one slice)", flush=True)
    dy = workloads.to_device(y)
    _check(xk, dy, 64, dy["limit"], "bf16 small")
    z = workloads.inputs("flash_decode")
    print("[no-alloc] flash_decode (decode batch)", flush=True)
    dz = workloads.to_device(z)
    _check(xk, dz, z["cfg"].topk, dz["limit"], "flash_decode")
