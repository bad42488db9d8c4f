"""The C ABI: library loads, exports every declared symbol, rejects bad
arguments on the host before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "xk.h")
LIB = os.path.join(ROOT, "sparse_attention_indexer_logits_amd", "libxk.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libxk.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(xk_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import sparse_attention_indexer_logits_amd as xk
    return xk.lib()


def test_header_declares_the_three_operations():
    names = declared_functions()
    for n in ("xk_indexer_logits", "xk_indexer_logits_paged", "xk_indexer_topk",
              "xk_indexer_logits_topk", "xk_indexer_logits_topk_workspace_size",
              "xk_sparse_attention_mxfp4",
              "xk_mxfp4_paged_gather", "xk_indexer_topk_workspace_size", "xk_quant_fp8_rows",
              "xk_mxfp4_cache_write", "xk_status_string", "xk_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(LIB)
    for n in declared_functions():
        assert hasattr(raw, n), n
    import sparse_attention_indexer_logits_amd as xk
    assert set(xk.EXPORTED) == set(declared_functions())


def test_status_strings(lib):
    assert lib.xk_status_string(0) == b"XK_OK"
    assert lib.xk_status_string(1) == b"XK_ERR_INVALID_ARGUMENT"
    assert lib.xk_status_string(2) == b"XK_ERR_UNSUPPORTED"
    assert lib.xk_status_string(3) == b"XK_ERR_HIP"


FAKE = 0x10000  # aligned, never dereferenced: validation fails before any HIP call


@pytest.mark.parametrize("args,status,needle", [
    # (q, q_scale, k, k_scale, w, limit, logits, B, T, K, H, D, dtype)
    ((None, None, FAKE, None, FAKE, None, FAKE, 1, 1, 8, 64, 128, 0), 1, "null"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 0, 1, 8, 64, 128, 0), 1, ">= 1"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 1, -3, 64, 128, 0), 1, ">= 1"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 1, 8, 64, 128, 7), 1, "dtype"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 1, 8, 64, 128, 1), 1, "scale"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 1, 8, 64, 128, 0), 1, "no scales"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 1, 8, 32, 128, 0), 2, "H=64"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 1, 8, 64, 64, 0), 2, "H=64"),
    ((FAKE + 2, None, FAKE, None, FAKE, None, FAKE, 1, 1, 8, 64, 128, 0), 1, "aligned"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1 << 16, 1 << 10, 1 << 20, 64, 128, 0), 2, "2^38"),
])
def test_logits_validation(lib, args, status, needle):
    assert lib.xk_indexer_logits(*args, None) == status
    assert needle in lib.xk_last_error().decode()


@pytest.mark.parametrize("args,status,needle", [
    # (q, q_scale, w, limit, k_cache, k_scale, block_table, logits,
    #  B, T, K, H, D, MB, NB, bs, kformat)
    ((FAKE, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 128, 1, 1, 64, 0), 1, "null"),
    ((FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 0, 64, 64, 128, 1, 1, 64, 0), 1, ">= 1"),
    ((FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 128, 1, 1, 64, 5), 1, "format"),
    ((FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 32, 128, 1, 1, 64, 0), 2, "H=64"),
    ((FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 128, 8, 1, 8, 0), 2, ">= 16"),
    ((FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 1, 48, 64, 128, 1, 1, 48, 1), 1, "power of two"),
    ((FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 1, 200, 64, 128, 3, 4, 64, 0), 1, "MB*bs"),
    ((FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 128, 1, 1 << 26, 64, 0), 2, "NB*bs"),
    ((FAKE, FAKE, FAKE, None, FAKE + 8, FAKE, FAKE, FAKE, 1, 1, 64, 64, 128, 1, 1, 64, 0), 1, "aligned"),
    ((FAKE, FAKE, FAKE, None, FAKE, FAKE + 2, FAKE, FAKE, 1, 1, 64, 64, 128, 1, 1, 64, 1), 1, "aligned"),
    ((FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 10, 1 << 10, 1 << 20, 64, 128, 1 << 14, 1, 64, 0), 2,
     "2^38"),
])
def test_logits_paged_validation(lib, args, status, needle):
    assert lib.xk_indexer_logits_paged(*args, None) == status
    assert needle in lib.xk_last_error().decode()


@pytest.mark.parametrize("args,status,needle", [
    # (logits, limit, idx, R, K, k, workspace, workspace_bytes)
    ((None, None, FAKE, 1, 8, 4, None, 0), 1, "null"),
    ((FAKE, None, FAKE, 0, 8, 4, None, 0), 1, ">= 1"),
    ((FAKE, None, FAKE, 1, 8, 0, None, 0), 1, ">= 1"),
    ((FAKE, None, FAKE, 1, 8, 4096, None, 0), 2, "2048"),
    ((FAKE, None, FAKE, 1, 8, -2, None, 0), 1, ">= 1"),
])
def test_topk_validation(lib, args, status, needle):
    assert lib.xk_indexer_topk(*args, None) == status
    assert needle in lib.xk_last_error().decode()


def test_topk_workspace_is_host_only(lib):
    assert lib.xk_indexer_topk_workspace_size(4096, 4096, 512) == 0


@pytest.mark.parametrize("args,status,needle", [
    # (q, q_scale, k, k_scale, w, limit, idx, B, T, K, H, D, topk, dtype, workspace, ws_bytes)
    ((None, None, FAKE, None, FAKE, None, FAKE, 1, 1, 8, 64, 128, 4, 0, FAKE, 1 << 20), 1, "null"),
    ((FAKE, None, FAKE, None, FAKE, None, None, 1, 1, 8, 64, 128, 4, 0, FAKE, 1 << 20), 1, "null"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 0, 8, 64, 128, 4, 0, FAKE, 1 << 20), 1, ">= 1"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 1, 8, 64, 128, 4, 1, FAKE, 1 << 20), 1, "scale"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 1, 8, 64, 64, 4, 0, FAKE, 1 << 20), 2, "H=64"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 1, 8, 64, 128, 0, 0, FAKE, 1 << 20), 1, "topk"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 1, 8, 64, 128, 4096, 0, FAKE, 1 << 20), 2, "2048"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 1, 8, 64, 128, 4, 0, None, 1 << 20), 1, "workspace"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 1, 8, 64, 128, 4, 0, FAKE, 16), 1, "workspace"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 1, 8, 64, 128, 4, 0, FAKE + 64, 1 << 20), 1, "256-byte"),
])
def test_logits_topk_validation(lib, args, status, needle):
    assert lib.xk_indexer_logits_topk(*args, None) == status
    assert needle in lib.xk_last_error().decode()


@pytest.mark.parametrize("args,status,needle", [
    # (q, q_scale, k, k_scale, w, limit, idx, B, T, K, H, D, topk, dtype); every case is
    # rejected on the host before any HIP call, so none of them touches the fake pointers
    ((None, None, FAKE, None, FAKE, None, FAKE, 1, 8, 64, 64, 128, 4, 0), 1, "null"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 8, 64, 64, 128, 0, 0), 1, ">= 1"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 8, 64, 64, 128, 4096, 0), 2, "2048"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 8, 64, 32, 128, 4, 0), 2, "H=64"),
    # a slice of 8 queries over 3M keys needs 96 MiB of scores: more than the built-in scratch
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 1, 8, 3 << 20, 64, 128, 512, 0), 2, "built-in scratch"),
    ((FAKE, None, FAKE, None, FAKE, None, FAKE, 4, 1, 20 << 20, 64, 128, 512, 0), 2, "built-in scratch"),
])
def test_logits_topk_noalloc_validation(lib, args, status, needle):
    assert lib.xk_indexer_logits_topk_noalloc(*args, None) == status
    assert needle in lib.xk_last_error().decode()


@pytest.mark.parametrize("args,status,needle", [
    # (q, kv_fp4, kv_scale, block_table, sel_pos, row_seq, sink, scale, out,
    #  R, H, k, S, MB, NB, bs, D)
    ((None, FAKE, FAKE, FAKE, FAKE, None, None, 1.0, FAKE, 1, 64, 4, 1, 1, 1, 64, 128), 1, "null"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 1.0, None, 1, 64, 4, 1, 1, 1, 64, 128), 1, "null"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 1.0, FAKE, 1, 64, 0, 1, 1, 1, 64, 128), 1, ">= 1"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, None, float("nan"), FAKE, 1, 64, 4, 1, 1, 1, 64, 128), 1, "finite"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 1.0, FAKE, 1, 64, 4, 1, 1, 1, 64, 64), 2, "D=128"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 1.0, FAKE, 1, 32, 4, 1, 1, 1, 64, 128), 2, "multiple of 64"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 1.0, FAKE, 1, 64, 4096, 1, 1, 1, 64, 128), 2, "2048"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 1.0, FAKE, 1, 64, 4, 1, 1, 1, 48, 128), 1, "power of two"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 1.0, FAKE, 3, 64, 4, 2, 1, 1, 64, 128), 1, "R <= S"),
    ((FAKE, FAKE + 4, FAKE, FAKE, FAKE, None, None, 1.0, FAKE, 1, 64, 4, 1, 1, 1, 64, 128), 1, "aligned"),
])
def test_sparse_attention_validation(lib, args, status, needle):
    assert lib.xk_sparse_attention_mxfp4(*args, None) == status
    assert needle in lib.xk_last_error().decode()


def test_logits_topk_workspace_sizes(lib):
    ws = lib.xk_indexer_logits_topk_workspace_size
    # rejected sizes report 0
    assert ws(1, 1, 8, 0, 0) == 0 and ws(1, 1, 8, 4096, 0) == 0 and ws(1, 1, 8, 4, 9) == 0
    assert ws(0, 1, 8, 4, 0) == 0
    # few queries: the score matrix itself (B*T*K fp32, 256-byte aligned)
    assert ws(32, 1, 8192, 512, 0) == 32 * 8192 * 4
    assert ws(1, 8, 100, 16, 0) == 3328
    # the long fp8 prefill shape: candidate regions (8 bytes x 16384 slots per
    # query) and 64 scratch rows, well under its 768 MiB score matrix
    big = ws(1, 2048, 98304, 1024, 1)
    assert 2048 * 16384 * 8 < big < 2048 * 98304 * 4 // 2
    # more keys per row leave the per-query room unchanged
    assert ws(1, 2048, 196608, 1024, 1) - big == 64 * 98304 * 4


@pytest.mark.parametrize("args,status,needle", [
    # (kv_fp4, kv_scale, block_table, sel_pos, row_seq, out, R, k, S, MB, NB, bs, D)
    ((None, FAKE, FAKE, FAKE, None, FAKE, 1, 4, 1, 1, 1, 64, 128), 1, "null"),
    ((FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 0, 1, 1, 1, 64, 128), 1, ">= 1"),
    ((FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 4, 1, 1, 1, 64, 64), 2, "D=128"),
    ((FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 4, 1, 1, 1, 48, 128), 1, "power of two"),
    ((FAKE, FAKE, FAKE, FAKE, None, FAKE, 3, 4, 2, 1, 1, 64, 128), 1, "R <= S"),
    ((FAKE + 1, FAKE, FAKE, FAKE, None, FAKE, 1, 4, 1, 1, 1, 64, 128), 1, "aligned"),
    ((FAKE, FAKE, FAKE, FAKE, None, FAKE + 4, 1, 4, 1, 1, 1, 64, 128), 1, "aligned"),
    ((FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 4, 1, 1, 1 << 26, 64, 128), 2, "NB*bs"),
])
def test_gather_validation(lib, args, status, needle):
    assert lib.xk_mxfp4_paged_gather(*args, None) == status
    assert needle in lib.xk_last_error().decode()


@pytest.mark.parametrize("args,status,needle", [
    # (x, x_dtype, out, scale, N, D)
    ((None, 0, FAKE, FAKE, 4, 128), 1, "null"),
    ((FAKE, 0, FAKE, FAKE, 0, 128), 1, ">= 1"),
    ((FAKE, 3, FAKE, FAKE, 4, 128), 1, "dtype"),
    ((FAKE, 0, FAKE, FAKE, 4, 64), 2, "D=128"),
    ((FAKE + 4, 0, FAKE, FAKE, 4, 128), 1, "misaligned"),
    ((FAKE, 0, FAKE, FAKE, (1 << 34) + 1, 128), 2, "2^34"),
])
def test_quant_fp8_rows_validation(lib, args, status, needle):
    assert lib.xk_quant_fp8_rows(*args, None) == status
    assert needle in lib.xk_last_error().decode()


@pytest.mark.parametrize("args,status,needle", [
    # (x, x_dtype, slots, kv_fp4, kv_scale, N, NB, bs, D)
    ((FAKE, 1, None, FAKE, FAKE, 4, 2, 64, 128), 1, "null"),
    ((FAKE, 1, FAKE, FAKE, FAKE, 4, 0, 64, 128), 1, ">= 1"),
    ((FAKE, 2, FAKE, FAKE, FAKE, 4, 2, 64, 128), 1, "dtype"),
    ((FAKE, 1, FAKE, FAKE, FAKE, 4, 2, 64, 256), 2, "D=128"),
    ((FAKE, 1, FAKE + 4, FAKE, FAKE, 4, 2, 64, 128), 1, "misaligned"),
    ((FAKE, 1, FAKE, FAKE, FAKE, (1 << 34) + 1, 2, 64, 128), 2, "2^34"),
])
def test_mxfp4_cache_write_validation(lib, args, status, needle):
    assert lib.xk_mxfp4_cache_write(*args, None) == status
    assert needle in lib.xk_last_error().decode()


def test_python_binding_rejects_host_tensors():
    import torch
    import sparse_attention_indexer_logits_amd as xk
    q = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        xk.xk_indexer_logits(q, torch.zeros((1, 8, 128), dtype=torch.bfloat16),
                             torch.zeros((1, 1, 64)))


def test_bench_probe_library_exports_and_checks_arguments():
    """The benchmark's achievable-rate probes (a library of their own, not the
    indexer ABI): exported, and bad arguments are refused before any launch."""
    path = os.path.join(ROOT, "sparse_attention_indexer_logits_amd", "libxk_peaks.so")
    if not os.path.exists(path):
        pytest.skip("libxk_peaks.so not built")
    raw = ctypes.CDLL(path)
    for n in ("xkp_device_info", "xkp_mfma_loop", "xkp_read_stream"):
        assert hasattr(raw, n), n
    raw.xkp_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
    raw.xkp_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert raw.xkp_mfma_loop(0, None, None, 16, 1, None) == 1          # no operand buffers
    assert raw.xkp_mfma_loop(0, 16, 16, 0, 1, None) == 1               # no workgroups
    assert raw.xkp_read_stream(8, 4, 16, 16, None) == 1                # source not 16-byte aligned
