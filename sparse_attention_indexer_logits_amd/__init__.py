"""Python binding of libxk, the MI355X (gfx950) DeepSeek-V4 DSA indexer path.

Thin ctypes marshalling over the C ABI declared in include/xk.h: each
function takes torch tensors, checks device/dtype/contiguity/shape, and calls
the C entry point of the same name on the current HIP stream. Every step of
the path runs in the HIP kernels of libxk.so; there is no other code path, and
importing this package fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libxk.so")

XK_OK, XK_ERR_INVALID_ARGUMENT, XK_ERR_UNSUPPORTED, XK_ERR_HIP = 0, 1, 2, 3
XK_BF16, XK_FP8_E4M3_OCP = 0, 1
XK_KCACHE_MXFP4, XK_KCACHE_FP8_E4M3_OCP = 0, 1
XK_IN_FP32, XK_IN_BF16 = 0, 1

EXPORTED = ("xk_indexer_logits", "xk_indexer_logits_paged", "xk_indexer_topk_workspace_size",
            "xk_indexer_topk", "xk_indexer_logits_topk_workspace_size", "xk_indexer_logits_topk",
            "xk_indexer_logits_topk_noalloc",
            "xk_mxfp4_paged_gather", "xk_sparse_attention_mxfp4", "xk_quant_fp8_rows", "xk_mxfp4_cache_write",
            "xk_status_string", "xk_last_error")


class XKError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_lib.xk_status_string(status).decode()}: {detail}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python sparse_attention_indexer_logits_amd/build.py` first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.xk_indexer_logits.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P]
    lib.xk_indexer_logits.restype = I
    lib.xk_indexer_logits_paged.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, P]
    lib.xk_indexer_logits_paged.restype = I
    lib.xk_indexer_topk_workspace_size.argtypes = [I, I, I]
    lib.xk_indexer_topk_workspace_size.restype = Z
    lib.xk_indexer_topk.argtypes = [P, P, P, I, I, I, P, Z, P]
    lib.xk_indexer_topk.restype = I
    lib.xk_indexer_logits_topk_workspace_size.argtypes = [I, I, I, I, I]
    lib.xk_indexer_logits_topk_workspace_size.restype = Z
    lib.xk_indexer_logits_topk.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, Z, P]
    lib.xk_indexer_logits_topk.restype = I
    lib.xk_indexer_logits_topk_noalloc.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P]
    lib.xk_indexer_logits_topk_noalloc.restype = I
    lib.xk_sparse_attention_mxfp4.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, P, I, I, I, I, I,
                                              I, I, I, P]
    lib.xk_sparse_attention_mxfp4.restype = I
    lib.xk_mxfp4_paged_gather.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, P]
    lib.xk_mxfp4_paged_gather.restype = I
    L = ctypes.c_int64
    lib.xk_quant_fp8_rows.argtypes = [P, I, P, P, L, I, P]
    lib.xk_quant_fp8_rows.restype = I
    lib.xk_mxfp4_cache_write.argtypes = [P, I, P, P, P, L, I, I, I, P]
    lib.xk_mxfp4_cache_write.restype = I
    lib.xk_status_string.argtypes = [I]
    lib.xk_status_string.restype = ctypes.c_char_p
    lib.xk_last_error.argtypes = []
    lib.xk_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _check(status: int) -> None:
    if status != XK_OK:
        raise XKError(status, _lib.xk_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t, name, dtypes, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor, got {tuple(t.shape)}")


def _logits_inputs(q, k, w, limit, q_scale, k_scale):
    """Check the score inputs shared by xk_indexer_logits and
    xk_indexer_logits_topk; returns (B, T, K, H, D, fp8)."""
    _need(q, "q", (torch.bfloat16, torch.float8_e4m3fn, torch.uint8), 4)
    B, T, H, D = q.shape
    fp8 = q.dtype != torch.bfloat16
    _need(k, "k", (q.dtype,), 3)
    K = k.shape[1]
    if k.shape[0] != B or k.shape[2] != D:
        raise ValueError("k must be [B,K,D]")
    _need(w, "w", (torch.float32,), 3)
    if tuple(w.shape) != (B, T, H):
        raise ValueError("w must be [B,T,H]")
    if limit is not None:
        _need(limit, "limit", (torch.int32,), 2)
        if tuple(limit.shape) != (B, T):
            raise ValueError("limit must be [B,T]")
    if fp8:
        _need(q_scale, "q_scale", (torch.float32,), 3)
        _need(k_scale, "k_scale", (torch.float32,), 2)
        if tuple(q_scale.shape) != (B, T, H) or tuple(k_scale.shape) != (B, K):
            raise ValueError("q_scale must be [B,T,H] and k_scale [B,K]")
    return B, T, K, H, D, fp8


def logits_args(q, k, w, limit=None, q_scale=None, k_scale=None, out=None):
    """Validate the arguments of xk_indexer_logits and return (C arguments
    without the stream, out). Callers that launch the same call repeatedly
    (IndexerStep) keep the tuple and skip re-validation."""
    B, T, K, H, D, fp8 = _logits_inputs(q, k, w, limit, q_scale, k_scale)
    if out is None:
        out = torch.empty((B, T, K), dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,), 3)
    if tuple(out.shape) != (B, T, K):
        raise ValueError("out must be [B,T,K]")
    args = (_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w), _ptr(limit), _ptr(out),
            B, T, K, H, D, XK_FP8_E4M3_OCP if fp8 else XK_BF16)
    return args, out


def xk_indexer_logits(q, k, w, limit=None, q_scale=None, k_scale=None, out=None, stream=None):
    """logits [B,T,K] fp32 = sum_h w * relu(q . k), -inf past limit (see include/xk.h).

    q [B,T,64,128] and k [B,K,128] are bfloat16, or float8_e4m3fn / uint8
    bytes with q_scale [B,T,64] and k_scale [B,K] fp32; w [B,T,64] fp32;
    limit [B,T] int32 or None.
    """
    args, out = logits_args(q, k, w, limit, q_scale, k_scale, out)
    _check(_lib.xk_indexer_logits(*args, _stream(stream)))
    return out


def logits_paged_args(q, q_scale, w, k_cache, k_scale, block_table, limit=None, K=None, out=None):
    """Validate the arguments of xk_indexer_logits_paged; returns (C arguments
    without the stream, out). The key format follows k_cache's dtype: uint8
    [NB,bs,64] is mxfp4 (k_scale uint8 [NB,bs,4]); float8_e4m3fn [NB,bs,128]
    is fp8 (k_scale float32 [NB,bs])."""
    _need(q, "q", (torch.float8_e4m3fn, torch.uint8), 4)
    B, T, H, D = q.shape
    _need(q_scale, "q_scale", (torch.float32,), 3)
    _need(w, "w", (torch.float32,), 3)
    if tuple(q_scale.shape) != (B, T, H) or tuple(w.shape) != (B, T, H):
        raise ValueError("q_scale and w must be [B,T,H]")
    _need(block_table, "block_table", (torch.int32,), 2)
    MB = block_table.shape[1]
    if block_table.shape[0] != B:
        raise ValueError("block_table must be [B,MB]")
    if k_cache.dtype == torch.uint8:
        fmt = XK_KCACHE_MXFP4
        _need(k_cache, "k_cache", (torch.uint8,), 3)
        NB, bs, half = k_cache.shape
        _need(k_scale, "k_scale", (torch.uint8,), 3)
        if 2 * half != D or tuple(k_scale.shape) != (NB, bs, D // 32):
            raise ValueError("mxfp4 k_cache must be [NB,bs,D/2] and k_scale [NB,bs,D/32]")
    else:
        fmt = XK_KCACHE_FP8_E4M3_OCP
        _need(k_cache, "k_cache", (torch.float8_e4m3fn,), 3)
        NB, bs, dk = k_cache.shape
        _need(k_scale, "k_scale", (torch.float32,), 2)
        if dk != D or tuple(k_scale.shape) != (NB, bs):
            raise ValueError("fp8 k_cache must be [NB,bs,D] and k_scale [NB,bs]")
    if K is None:
        K = MB * bs
    if limit is not None:
        _need(limit, "limit", (torch.int32,), 2)
        if tuple(limit.shape) != (B, T):
            raise ValueError("limit must be [B,T]")
    if out is None:
        out = torch.empty((B, T, K), dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,), 3)
    if tuple(out.shape) != (B, T, K):
        raise ValueError("out must be [B,T,K]")
    args = (_ptr(q), _ptr(q_scale), _ptr(w), _ptr(limit), _ptr(k_cache), _ptr(k_scale),
            _ptr(block_table), _ptr(out), B, T, K, H, D, MB, NB, bs, fmt)
    return args, out


def xk_indexer_logits_paged(q, q_scale, w, k_cache, k_scale, block_table, limit=None, K=None,
                            out=None, stream=None):
    """logits [B,T,K] fp32 with keys in a paged mxfp4 / fp8 cache (see include/xk.h)."""
    args, out = logits_paged_args(q, q_scale, w, k_cache, k_scale, block_table, limit, K, out)
    _check(_lib.xk_indexer_logits_paged(*args, _stream(stream)))
    return out


def xk_indexer_topk_workspace_size(R: int, K: int, k: int) -> int:
    return int(_lib.xk_indexer_topk_workspace_size(R, K, k))


def topk_args(logits, k: int, limit=None, out=None, workspace=None):
    """Validate the arguments of xk_indexer_topk; returns (C arguments without
    the stream, out, workspace)."""
    if logits.dim() == 3:
        logits = logits.view(-1, logits.shape[-1])
    _need(logits, "logits", (torch.float32,), 2)
    R, K = logits.shape
    if limit is not None:
        limit = limit.reshape(-1)
        _need(limit, "limit", (torch.int32,), 1)
        if limit.shape[0] != R:
            raise ValueError("limit must have R entries")
    if out is None:
        out = torch.empty((R, k), dtype=torch.int32, device=logits.device)
    _need(out, "out", (torch.int32,), 2)
    if tuple(out.shape) != (R, k):
        raise ValueError("out must be [R,k]")
    need = xk_indexer_topk_workspace_size(R, K, k)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace is not None and workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small")
    return (_ptr(logits), _ptr(limit), _ptr(out), R, K, k, _ptr(workspace), ws_bytes), out, workspace


def xk_indexer_topk(logits, k: int, limit=None, out=None, workspace=None, stream=None):
    """idx [R,k] int32: top-k per row by (score desc, j asc), -1 padded (see include/xk.h).

    logits [R,K] fp32 (a [B,T,K] tensor is viewed as [B*T,K]); limit [R] int32 or None.
    """
    args, out, _ = topk_args(logits, k, limit, out, workspace)
    _check(_lib.xk_indexer_topk(*args, _stream(stream)))
    return out


def xk_indexer_logits_topk_workspace_size(B: int, T: int, K: int, k: int, dtype: int) -> int:
    return int(_lib.xk_indexer_logits_topk_workspace_size(B, T, K, k, dtype))


def logits_topk_args(q, k, w, topk: int, limit=None, q_scale=None, k_scale=None, out=None,
                     workspace=None):
    """Validate the arguments of xk_indexer_logits_topk; returns (C arguments
    without the stream, out, workspace). A workspace of the size the library
    asks for is allocated when none is given."""
    B, T, K, H, D, fp8 = _logits_inputs(q, k, w, limit, q_scale, k_scale)
    dtype = XK_FP8_E4M3_OCP if fp8 else XK_BF16
    if out is None:
        out = torch.empty((B * T, topk), dtype=torch.int32, device=q.device)
    _need(out, "out", (torch.int32,), 2)
    if tuple(out.shape) != (B * T, topk):
        raise ValueError("out must be [B*T,topk]")
    need = xk_indexer_logits_topk_workspace_size(B, T, K, topk, dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    if ws_bytes < need:
        raise ValueError("workspace too small")
    args = (_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w), _ptr(limit), _ptr(out),
            B, T, K, H, D, topk, dtype, _ptr(workspace), ws_bytes)
    return args, out, workspace


def xk_indexer_logits_topk(q, k, w, topk: int, limit=None, q_scale=None, k_scale=None, out=None,
                           workspace=None, stream=None):
    """idx [B*T,topk] int32 = xk_indexer_topk(xk_indexer_logits(...)), without the
    score matrix for prefill shapes (see include/xk.h). Inputs as for
    xk_indexer_logits."""
    args, out, _ = logits_topk_args(q, k, w, topk, limit, q_scale, k_scale, out, workspace)
    _check(_lib.xk_indexer_logits_topk(*args, _stream(stream)))
    return out


def xk_indexer_logits_topk_noalloc(q, k, w, topk: int, limit=None, q_scale=None, k_scale=None, out=None,
                                   stream=None):
    """xk_indexer_logits_topk without a workspace: the library's built-in
    scratch (see include/xk.h). Same result; `out` is the only buffer."""
    B, T, K, H, D, fp8 = _logits_inputs(q, k, w, limit, q_scale, k_scale)
    if out is None:
        out = torch.empty((B * T, topk), dtype=torch.int32, device=q.device)
    _need(out, "out", (torch.int32,), 2)
    if tuple(out.shape) != (B * T, topk):
        raise ValueError("out must be [B*T,topk]")
    dtype = XK_FP8_E4M3_OCP if fp8 else XK_BF16
    _check(_lib.xk_indexer_logits_topk_noalloc(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w),
                                               _ptr(limit), _ptr(out), B, T, K, H, D, topk, dtype,
                                               _stream(stream)))
    return out


def gather_args(kv_fp4, kv_scale, block_table, sel_pos, row_seq=None, out=None):
    """Validate the arguments of xk_mxfp4_paged_gather; returns (C arguments
    without the stream, out)."""
    _need(kv_fp4, "kv_fp4", (torch.uint8,), 3)
    NB, bs, half = kv_fp4.shape
    D = 2 * half
    _need(kv_scale, "kv_scale", (torch.uint8,), 3)
    if tuple(kv_scale.shape) != (NB, bs, D // 32):
        raise ValueError("kv_scale must be [NB,bs,D/32]")
    _need(block_table, "block_table", (torch.int32,), 2)
    S, MB = block_table.shape
    _need(sel_pos, "sel_pos", (torch.int32,), 2)
    R, k = sel_pos.shape
    if row_seq is not None:
        _need(row_seq, "row_seq", (torch.int32,), 1)
        if row_seq.shape[0] != R:
            raise ValueError("row_seq must have R entries")
    if out is None:
        out = torch.empty((R, k, D), dtype=torch.int16, device=kv_fp4.device)
    _need(out, "out", (torch.int16, torch.bfloat16), 3)
    if tuple(out.shape) != (R, k, D):
        raise ValueError("out must be [R,k,D]")
    args = (_ptr(kv_fp4), _ptr(kv_scale), _ptr(block_table), _ptr(sel_pos), _ptr(row_seq),
            _ptr(out), R, k, S, MB, NB, bs, D)
    return args, out


def xk_mxfp4_paged_gather(kv_fp4, kv_scale, block_table, sel_pos, row_seq=None, out=None,
                          stream=None):
    """out [R,k,128] bf16 bits (int16 storage) of the selected mxfp4 rows (see include/xk.h).

    kv_fp4 [NB,bs,64] uint8; kv_scale [NB,bs,4] uint8; block_table [S,MB] int32;
    sel_pos [R,k] int32; row_seq [R] int32 or None.
    """
    args, out = gather_args(kv_fp4, kv_scale, block_table, sel_pos, row_seq, out)
    _check(_lib.xk_mxfp4_paged_gather(*args, _stream(stream)))
    return out


def attention_args(q, kv_fp4, kv_scale, block_table, sel_pos, row_seq=None, sink=None, scale=None,
                   out=None):
    """Validate the arguments of xk_sparse_attention_mxfp4; returns (C
    arguments without the stream, out). scale None means 1/sqrt(D)."""
    _need(q, "q", (torch.bfloat16,), 3)
    R, H, D = q.shape
    _need(kv_fp4, "kv_fp4", (torch.uint8,), 3)
    _need(kv_scale, "kv_scale", (torch.uint8,), 3)
    NB, bs, half = kv_fp4.shape
    if 2 * half != D or tuple(kv_scale.shape) != (NB, bs, D // 32):
        raise ValueError("kv_fp4 must be [NB,bs,D/2] and kv_scale [NB,bs,D/32]")
    _need(block_table, "block_table", (torch.int32,), 2)
    S, MB = block_table.shape
    _need(sel_pos, "sel_pos", (torch.int32,), 2)
    if sel_pos.shape[0] != R:
        raise ValueError("sel_pos must be [R,k]")
    k = sel_pos.shape[1]
    if row_seq is not None:
        _need(row_seq, "row_seq", (torch.int32,), 1)
        if row_seq.shape[0] != R:
            raise ValueError("row_seq must have R entries")
    if sink is not None:
        _need(sink, "sink", (torch.float32,), 1)
        if sink.shape[0] != H:
            raise ValueError("sink must have H entries")
    if scale is None:
        scale = 1.0 / D ** 0.5
    if out is None:
        out = torch.empty((R, H, D), dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,), 3)
    if tuple(out.shape) != (R, H, D):
        raise ValueError("out must be [R,H,D]")
    args = (_ptr(q), _ptr(kv_fp4), _ptr(kv_scale), _ptr(block_table), _ptr(sel_pos), _ptr(row_seq),
            _ptr(sink), float(scale), _ptr(out), R, H, k, S, MB, NB, bs, D)
    return args, out


def xk_sparse_attention_mxfp4(q, kv_fp4, kv_scale, block_table, sel_pos, row_seq=None, sink=None,
                              scale=None, out=None, stream=None):
    """out [R,H,D] fp32: attention of each query over its selected mxfp4 cache
    rows with a per-head sink logit (see include/xk.h)."""
    args, out = attention_args(q, kv_fp4, kv_scale, block_table, sel_pos, row_seq, sink, scale, out)
    _check(_lib.xk_sparse_attention_mxfp4(*args, _stream(stream)))
    return out


def _rows_in(x, name):
    _need(x, name, (torch.float32, torch.bfloat16), 2)
    return XK_IN_BF16 if x.dtype == torch.bfloat16 else XK_IN_FP32


def xk_quant_fp8_rows(x, out=None, scale=None, stream=None):
    """(codes [N,D] float8_e4m3fn, scale [N] fp32) of rows x [N,D] fp32/bf16
    (see include/xk.h): scale = amax/448, codes = e4m3(x/scale)."""
    dt = _rows_in(x, "x")
    N, D = x.shape
    if out is None:
        out = torch.empty((N, D), dtype=torch.float8_e4m3fn, device=x.device)
    if scale is None:
        scale = torch.empty((N,), dtype=torch.float32, device=x.device)
    _need(out, "out", (torch.float8_e4m3fn, torch.uint8), 2)
    _need(scale, "scale", (torch.float32,), 1)
    if tuple(out.shape) != (N, D) or scale.shape[0] != N:
        raise ValueError("out must be [N,D] and scale [N]")
    _check(_lib.xk_quant_fp8_rows(_ptr(x), dt, _ptr(out), _ptr(scale), N, D, _stream(stream)))
    return out, scale


def xk_mxfp4_cache_write(x, slots, kv_fp4, kv_scale, stream=None):
    """Write rows x [N,D] fp32/bf16 into the paged mxfp4 cache at slots [N]
    int64 (page * bs + row; < 0 skips), in place (see include/xk.h)."""
    dt = _rows_in(x, "x")
    N, D = x.shape
    _need(slots, "slots", (torch.int64,), 1)
    _need(kv_fp4, "kv_fp4", (torch.uint8,), 3)
    _need(kv_scale, "kv_scale", (torch.uint8,), 3)
    NB, bs, half = kv_fp4.shape
    if slots.shape[0] != N or 2 * half != D or tuple(kv_scale.shape) != (NB, bs, D // 32):
        raise ValueError("slots [N], kv_fp4 [NB,bs,D/2], kv_scale [NB,bs,D/32] expected")
    _check(_lib.xk_mxfp4_cache_write(_ptr(x), dt, _ptr(slots), _ptr(kv_fp4), _ptr(kv_scale), N,
                                     NB, bs, D, _stream(stream)))
    return kv_fp4, kv_scale
