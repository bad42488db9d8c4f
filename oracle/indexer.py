"""The three indexer operations, written from their definitions in float64.

Sources (pages, not code):
  [P27] "xkernels #27 -- [AMD/MI300A] DeepSeek-V4 DSA indexer + attention",
        comment "What shipped": the indexer score
        logits[t,j] = sum_h w[t,h] * relu(q[t,h,:] . k[j,:]) with q [T,H,D],
        one shared MQA key k [K,D], per-head weights, optional causal window,
        bf16/fp16 in and fp32 logits out; fp8/fp4 packing is an encoding of
        the same dequantized math.
  [P28] "xkernels #28 -- [AMD/MI300A] DeepSeek-V4 serving support", comment
        shipping mxfp4_paged_gather: per (seq, top-k slot) look up the block
        table, decode E2M1 nibbles times the E8M0 group scale 2**(b-127)
        (0xFF -> 0) broadcast over the group, bf16 out, sel_pos < 0 -> zero row;
        the selection is top-512 (Flash) / top-1024 (Pro).
  [PMX] "DeepSeek V4 Flash on a single AMD MI300X", overlay table and
        "Prefill" section: deterministic sparse top-k with a tie-break, and a
        canonical sort of the selected top-k.

Readings where the pages are silent (each also listed in the design notes):
  * the causal window is an inclusive upper bound j <= limit[b,t]; masked
    entries are exactly -inf; no scaling constant inside the score;
  * top-k order is (score descending, then lower j), -0.0 == +0.0, padded
    with -1 when fewer than k keys are valid;
  * mxfp4 byte layout: kv_fp4 [NB, bs, D/2] with element 2i in the low nibble,
    kv_scale [NB, bs, D/32], group g covering d in [32g, 32g+32);
  * logits from a paged quantized key cache compute the same score on the
    dequantized keys, the mxfp4 keys decoded exactly as the gather decodes
    them (E8M0 0xFF -> 0 included).
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, e4m3_to_f64, e2m1_to_f64, e8m0_to_f64, f64_to_bf16_bits


# ----------------------------------------------------------------------------- logits
def dequant_q(q, q_scale, dtype):
    """q_hat [B,T,H,D] float64: bf16 bits, or e4m3 code times its (t,h) scale."""
    if dtype == "bf16":
        return bf16_bits_to_f64(q)
    return e4m3_to_f64(q) * np.asarray(q_scale, dtype=np.float64)[..., None]


def dequant_k(k, k_scale, dtype):
    """k_hat [B,K,D] float64: bf16 bits, or e4m3 code times its per-token scale."""
    if dtype == "bf16":
        return bf16_bits_to_f64(k)
    return e4m3_to_f64(k) * np.asarray(k_scale, dtype=np.float64)[..., None]


def indexer_logits(q, k, w, limit=None, q_scale=None, k_scale=None, dtype="bf16",
                   rows=None):
    """Indexer logits [B,T,K] float32 [P27].

    q: [B,T,H,D] bf16 bits (uint16) or e4m3 bytes; k: [B,K,D] likewise;
    w: [B,T,H] float32; limit: [B,T] int32 inclusive last valid key (None:
    every key valid).  Each valid score is summed in float64 and rounded once
    to float32; masked entries are -inf.  ``rows`` optionally restricts the
    work to a list of (b, t) pairs (other rows are left NaN).
    """
    B, T, H, D = q.shape
    K = k.shape[1]
    w64 = np.asarray(w, dtype=np.float64)
    out = np.full((B, T, K), np.nan, dtype=np.float32)
    todo = rows if rows is not None else [(b, t) for b in range(B) for t in range(T)]
    by_seq = {}
    for b, t in todo:
        by_seq.setdefault(int(b), []).append(int(t))
    for b, ts in by_seq.items():
        # dequantize only this sequence (and only up to its furthest valid key)
        lims = [K - 1 if limit is None else int(limit[b, t]) for t in ts]
        n_max = max(0, min(max(lims) + 1, K))
        k_hat = dequant_k(k[b: b + 1, :n_max], None if k_scale is None else k_scale[b: b + 1, :n_max],
                          dtype)[0]
        for t, lim in zip(ts, lims):
            n = max(0, min(lim + 1, K))
            q_hat = dequant_q(q[b: b + 1, t: t + 1],
                              None if q_scale is None else q_scale[b: b + 1, t: t + 1], dtype)[0, 0]
            row = np.full(K, -np.inf, dtype=np.float64)
            if n:
                dots = q_hat @ k_hat[:n].T                   # [H, n]
                row[:n] = np.sum(w64[b, t][:, None] * np.maximum(dots, 0.0), axis=0)
            out[b, t] = row.astype(np.float32)
    return out


# ----------------------------------------------------------------------------- paged keys
def paged_keys(k_cache, k_scale, block_table, b, n, block_size, kfmt):
    """k_hat [n,D] float64: the first n logical keys of sequence b, read
    through its block table (position p -> block_table[b, p // bs], row
    p % bs) and dequantized.

    kfmt "mxfp4": k_cache [NB,bs,D/2] E2M1 nibbles (element 2i low),
                  k_scale [NB,bs,D/32] E8M0 bytes (0xFF -> 0), group g = d in
                  [32g, 32g+32) -- the cache format of the mxfp4 gather [P28];
    kfmt "fp8":   k_cache [NB,bs,D] OCP e4m3 bytes, k_scale [NB,bs] float32
                  per-token scale (the fp8 key encoding of the dense logits).
    """
    p = np.arange(n, dtype=np.int64)
    blk = np.asarray(block_table, dtype=np.int64)[b, p // block_size]
    off = p % block_size
    if kfmt == "mxfp4":
        packed = np.asarray(k_cache)[blk, off].astype(np.int64)       # [n, D/2]
        D = packed.shape[-1] * 2
        nib = np.empty((n, D), dtype=np.int64)
        nib[:, 0::2] = packed & 0xF
        nib[:, 1::2] = packed >> 4
        scale = e8m0_to_f64(np.asarray(k_scale)[blk, off])             # [n, D/32]
        return e2m1_to_f64(nib) * np.repeat(scale, D // scale.shape[-1], axis=-1)
    if kfmt == "fp8":
        codes = np.asarray(k_cache)[blk, off]
        return e4m3_to_f64(codes) * np.asarray(k_scale, dtype=np.float64)[blk, off][:, None]
    raise ValueError(kfmt)


def indexer_logits_paged(q, q_scale, w, limit, k_cache, k_scale, block_table, block_size, K,
                         kfmt="mxfp4", rows=None):
    """Indexer logits [B,T,K] float32 with keys in a paged quantized cache.

    The same score as indexer_logits [P27] ("fp8/fp4 packing" is an encoding
    of the dequantized math): q is OCP e4m3 [B,T,H,D] with q_scale [B,T,H];
    key j of sequence b is paged_keys(...)[j]; K is the logical key count of
    the output rows.  Float64 sums, one rounding to float32, -inf past the
    limit.  ``rows`` restricts the work to (b, t) pairs (others left NaN).
    """
    B, T, H, D = q.shape
    w64 = np.asarray(w, dtype=np.float64)
    out = np.full((B, T, K), np.nan, dtype=np.float32)
    todo = rows if rows is not None else [(b, t) for b in range(B) for t in range(T)]
    by_seq = {}
    for b, t in todo:
        by_seq.setdefault(int(b), []).append(int(t))
    for b, ts in by_seq.items():
        lims = [K - 1 if limit is None else int(limit[b, t]) for t in ts]
        n_max = max(0, min(max(lims) + 1, K))
        k_hat = paged_keys(k_cache, k_scale, block_table, b, n_max, block_size, kfmt)
        for t, lim in zip(ts, lims):
            n = max(0, min(lim + 1, K))
            q_hat = dequant_q(q[b: b + 1, t: t + 1], q_scale[b: b + 1, t: t + 1], "fp8")[0, 0]
            row = np.full(K, -np.inf, dtype=np.float64)
            if n:
                dots = q_hat @ k_hat[:n].T                   # [H, n]
                row[:n] = np.sum(w64[b, t][:, None] * np.maximum(dots, 0.0), axis=0)
            out[b, t] = row.astype(np.float32)
    return out


# ----------------------------------------------------------------------------- top-k
def topk_row(scores, n_valid, k):
    """Top-k of one row [P28 sizes, PMX tie-break and canonical order].

    Among j < n_valid, the min(k, n_valid) largest scores ordered by
    (score descending, j ascending); -0.0 counts as +0.0; remaining slots -1.
    """
    s = np.asarray(scores, dtype=np.float32)[: max(0, n_valid)].astype(np.float64)
    if np.isnan(s).any():
        raise ValueError("NaN score: outside the top-k contract")
    s = np.where(s == 0.0, 0.0, s)              # -0.0 -> +0.0
    j = np.arange(s.size)
    order = np.lexsort((j, -s))                  # primary: -score ascending; then j ascending
    m = min(k, s.size)
    out = np.full(k, -1, dtype=np.int32)
    out[:m] = order[:m]
    return out


def indexer_topk(logits, limit, k, rows=None):
    """Top-k indices [R,k] int32 for logits [R,K]; limit [R] (None: all valid)."""
    R, K = logits.shape
    out = np.full((R, k), -1, dtype=np.int32)
    for r in (range(R) if rows is None else rows):
        n = K if limit is None else max(0, min(int(limit[r]) + 1, K))
        out[r] = topk_row(logits[r], n, k)
    return out


# ----------------------------------------------------------------------------- gather
def mxfp4_paged_gather(kv_fp4, kv_scale, block_table, sel_pos, row_seq, block_size,
                       rows=None):
    """mxfp4 paged gather -> bf16 bits [R,k,D] (uint16) [P28].

    For slot (r, s) with p = sel_pos[r, s]:
      p < 0  -> a row of +0.0;
      else   -> blk = block_table[row_seq[r], p // bs], off = p % bs, and
                out[d] = bf16(E2M1(nibble d) * E8M0(scale byte d // 32)).
    The product is exact in float64 and rounded once to bf16.  ``rows``
    optionally restricts the work to a list of rows (others left 0xFFFF).
    """
    sel_all = np.asarray(sel_pos, dtype=np.int64)
    R, k = sel_all.shape
    D = kv_fp4.shape[2] * 2
    out = np.full((R, k, D), 0xFFFF, dtype=np.uint16)
    todo = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    for lo in range(0, todo.size, 256):          # row chunks only bound host memory
        r = todo[lo: lo + 256]
        out[r] = _gather_rows(kv_fp4, kv_scale, block_table, sel_all[r],
                              np.asarray(row_seq, dtype=np.int64)[r], block_size)
    return out


def _gather_rows(kv_fp4, kv_scale, block_table, sel, seq_of_row, block_size):
    R, k = sel.shape
    D = kv_fp4.shape[2] * 2
    G = kv_scale.shape[2]
    gsize = D // G
    seq = seq_of_row[:, None].repeat(k, axis=1)
    valid = sel >= 0
    p = np.where(valid, sel, 0)
    blk = np.asarray(block_table, dtype=np.int64)[seq, p // block_size]
    off = p % block_size
    packed = kv_fp4[blk, off].astype(np.int64)               # [R,k,D/2]
    nib = np.empty(packed.shape[:-1] + (D,), dtype=np.int64)
    nib[..., 0::2] = packed & 0xF                             # element 2i: low nibble
    nib[..., 1::2] = packed >> 4                              # element 2i+1: high nibble
    scale = e8m0_to_f64(kv_scale[blk, off])                   # [R,k,G]
    vals = e2m1_to_f64(nib) * np.repeat(scale, gsize, axis=-1)
    bits = f64_to_bf16_bits(vals)
    bits[~valid] = 0
    return bits
