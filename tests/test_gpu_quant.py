"""Parity of the producers (xk_quant_fp8_rows, xk_mxfp4_cache_write) with the
oracle, bit for bit, through the C ABI: codes and scales decided from the
same float32 values on both sides."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def xk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_logits_amd as xk
    return xk


def _rows(seed, N):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((N, 128)) * np.exp2(rng.integers(-20, 20, (N, 1)))).astype(np.float32)
    if N > 8:
        x[1] = 0.0                                      # all-zero row
        x[2] = -0.0
        x[3, :64] = 0.0                                 # zero half
        # amax 448 -> scale 1: exact e4m3 midpoints (ties to even) and subnormals
        pos = np.sort(oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8)))
        mids = ((pos[1:] + pos[:-1]) / 2)
        x[4] = np.resize(np.r_[448.0, mids[::-1]], 128) * np.where(np.arange(128) % 2, -1, 1)
        x[5] = np.r_[448.0, rng.uniform(-2 ** -6, 2 ** -6, 127)]
        # E2M1 midpoints inside groups of amax 6 (e = 0) and saturation (amax 7.5)
        x[6] = np.resize([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 5.5, 0.1], 128)
        x[7, :32] = 7.5
        x[7, 32:] = np.resize([1e-30, -3e-38, 2e-40], 96)  # tiny groups (subnormal range)
    if N > 10:
        # scale 3 (amax 1344): quotients that are exact e4m3 midpoints at a scale that is not a
        # power of two, so ties reach the encoder through a rounded division
        pos = np.sort(oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8)))
        mids = (pos[1:] + pos[:-1]) / 2
        x[8] = np.resize(np.r_[1344.0, 3 * mids[::-1]], 128) * np.where(np.arange(128) % 2, -1, 1)
        # a subnormal scale (amax 1e-37): the rounded scale puts |x / scale| just above 448
        x[9] = np.r_[1e-37, np.linspace(-1e-37, 1e-37, 127)]
    return x


# (1 << 20) + 3 rows: the fp8 launch shape for many rows (two passes per wave), ragged
@pytest.mark.parametrize("dtype,N", [(d, n) for d in ("fp32", "bf16") for n in (1, 7, 1000, 98304)]
                         + [("fp32", (1 << 20) + 3)])
def test_quant_fp8_rows(xk, dtype, N):
    x = _rows(N, N)
    xt = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
        x = xt.float().cpu().numpy()                # the oracle quantizes the bf16 values
    print(f"[quant] fp8 rows dtype={dtype} N={N}", flush=True)
    out = torch.full((N, 128), 0x7F, dtype=torch.uint8, device="cuda")
    scale = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    xk.xk_quant_fp8_rows(xt, out=out, scale=scale)
    torch.cuda.synchronize()
    codes, sc = oracle.quant_fp8_rows(x)
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), sc.view(np.uint32))
    assert np.array_equal(out.cpu().numpy(), codes)


@pytest.mark.parametrize("dtype,N,NB,bs", [(d, n, nb, bs) for d in ("fp32", "bf16")
                                           for n, nb, bs in ((5, 2, 16), (300, 8, 64), (98304, 1536, 64))]
                         + [("bf16", (1 << 20) + 3, 16400, 64)])
def test_mxfp4_cache_write(xk, dtype, N, NB, bs):
    rng = np.random.default_rng(N)
    x = _rows(N + 1, N)
    xt = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
        x = xt.float().cpu().numpy()
    total = NB * bs
    slots = rng.permutation(max(total, N))[:N].astype(np.int64)
    slots[slots >= total] = -1                      # rows with no slot are skipped
    if N > 3:
        slots[0] = -1
        slots[2] = total + 5                        # out of range: skipped too
    print(f"[quant] mxfp4 write dtype={dtype} N={N} NB={NB} bs={bs}", flush=True)
    kv0 = rng.integers(0, 256, (NB, bs, 64), dtype=np.uint8)   # stale contents stay where not written
    sc0 = rng.integers(0, 256, (NB, bs, 4), dtype=np.uint8)
    kv, sc = torch.from_numpy(kv0).cuda(), torch.from_numpy(sc0).cuda()
    xk.xk_mxfp4_cache_write(xt, torch.from_numpy(slots).cuda(), kv, sc)
    torch.cuda.synchronize()
    slots_o = np.where(slots < total, slots, -1)
    ref_kv, ref_sc = oracle.mxfp4_cache_write(x, slots_o, kv0, sc0)
    assert np.array_equal(kv.cpu().numpy(), ref_kv)
    assert np.array_equal(sc.cpu().numpy(), ref_sc)


def test_write_then_gather_round_trip(xk):
    """GPU writer -> GPU gather equals oracle writer -> oracle gather."""
    rng = np.random.default_rng(4)
    N, NB, bs = 256, 8, 64
    x = _rows(9, N)
    slots = rng.permutation(NB * bs)[:N].astype(np.int64)
    kv = torch.zeros((NB, bs, 64), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((NB, bs, 4), dtype=torch.uint8, device="cuda")
    xk.xk_mxfp4_cache_write(torch.from_numpy(x).cuda(), torch.from_numpy(slots).cuda(), kv, sc)
    table = torch.arange(NB, dtype=torch.int32, device="cuda")[None, :]
    sel = torch.from_numpy(slots.astype(np.int32))[None, :].cuda()
    g = xk.xk_mxfp4_paged_gather(kv, sc, table, sel).cpu().numpy().view(np.uint16)
    rk, rs = oracle.mxfp4_cache_write(x, slots, np.zeros((NB, bs, 64), np.uint8), np.zeros((NB, bs, 4), np.uint8))
    o = oracle.mxfp4_paged_gather(rk, rs, np.arange(NB, dtype=np.int32)[None, :], slots.astype(np.int32)[None, :],
                                  np.zeros(1, np.int32), bs)
    assert np.array_equal(g, o)
