"""Producers of the path's quantized inputs, written from their definitions.

Sources (pages, not code):
  [PMX] "DeepSeek V4 Flash on a single AMD MI300X", "FP8 format" fix: the
        indexer's fp8 cache is OCP e4m3 written with FP8_MAX = 448.
  [PVL] "[ROCm][DSv4][WIP] Sparse-MLA bring-up on MI300X": the compressed-K
        and indexer-Q writers quantize with FP8_MAX = 448 (OCP) per row.
  [PAT] "DeepSeek-V4 on ATOM" tracker, "Quantization & Transform": act_quant
        BF16 -> FP8 e4m3 per 1x128 block.
  [P28] "xkernels #28 -- DeepSeek-V4 serving support", comment shipping
        mxfp4_paged_gather: the paged mxfp4 cache (E2M1 nibbles, E8M0 group
        scale 2^(b-127)) whose reader the gather is.

Readings where the pages are silent (also listed in the design notes):
  * fp8 rows: scale = amax / 448 in float32 (1.0 for an all-zero row),
    code = round-to-nearest-even e4m3 of the float32 quotient x / scale,
    saturated to +-448;
  * mxfp4 writer (the OCP MX rule): per 32-element group, exponent e =
    floor(log2(amax)) - 2 (E2M1's largest exponent), clamped to
    [-127, 127] (an all-zero group gets -127), E8M0 byte e + 127; element =
    round-to-nearest-even E2M1 of the float32 x * 2^-e, saturated to +-6;
    element 2i in the low nibble.
Integer codes are decided from float32 values, as the kernels decide them.
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_to_f64, e2m1_to_f64

FP8_MAX = 448.0


def _nearest_even_code(v, codes, values):
    """Code of the representable value nearest |v| (ties to the even code:
    the one whose mantissa bit is 0); ``values`` ascending, non-negative."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    hi = np.clip(np.searchsorted(values, a, side="left"), 0, values.size - 1)
    lo = np.clip(hi - 1, 0, values.size - 1)
    d_lo, d_hi = a - values[lo], values[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    return np.where(pick_hi, codes[hi], codes[lo])


_E4M3_POS = np.arange(0x7F, dtype=np.int64)          # 0x00..0x7E: +0 .. 448 (0x7F is NaN)
_E4M3_VAL = e4m3_to_f64(_E4M3_POS.astype(np.uint8))
_E2M1_POS = np.arange(8, dtype=np.int64)              # +0 .. 6
_E2M1_VAL = e2m1_to_f64(_E2M1_POS)


def e4m3_encode(v) -> np.ndarray:
    """float -> OCP e4m3 byte, round to nearest even, saturated to +-448."""
    v = np.asarray(v, dtype=np.float64)
    mag = _nearest_even_code(np.minimum(np.abs(v), FP8_MAX), _E4M3_POS, _E4M3_VAL)
    return (mag | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def e2m1_encode(v) -> np.ndarray:
    """float -> E2M1 nibble, round to nearest even, saturated to +-6."""
    v = np.asarray(v, dtype=np.float64)
    mag = _nearest_even_code(np.minimum(np.abs(v), 6.0), _E2M1_POS, _E2M1_VAL)
    return (mag | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def quant_fp8_rows(x):
    """x [N,D] float32 -> (codes [N,D] uint8 OCP e4m3, scale [N] float32).

    Per row (a token's key, or a token's head of q): scale = amax / 448 in
    float32, 1.0 when the row is all zero; codes = e4m3(x / scale) with the
    quotient rounded to float32 first.
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    q = (x / scale[..., None]).astype(np.float32)
    return e4m3_encode(q), scale


def mxfp4_encode_rows(x):
    """x [N,D] float32 -> (packed [N,D/2] uint8 E2M1 nibbles, scale [N,D/32] uint8 E8M0)."""
    x = np.asarray(x, dtype=np.float32)
    N, D = x.shape
    g = x.reshape(N, D // 32, 32)
    amax = np.abs(g).max(axis=-1).astype(np.float64)
    _, ex = np.frexp(amax)                                  # amax = m * 2^ex, m in [0.5, 1)
    e = np.where(amax > 0, ex - 1 - 2, -127)
    e = np.clip(e, -127, 127)
    v = (g * np.ldexp(np.float32(1.0), -e)[..., None].astype(np.float32)).astype(np.float32)
    nib = e2m1_encode(v).reshape(N, D).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def mxfp4_cache_write(x, slots, kv_fp4, kv_scale):
    """Write rows x [N,D] into the paged cache at physical slots [N] (slot =
    block * bs + offset; negative slots are skipped); returns new arrays."""
    kv_fp4 = np.array(kv_fp4, copy=True)
    kv_scale = np.array(kv_scale, copy=True)
    NB, bs = kv_fp4.shape[:2]
    packed, sc = mxfp4_encode_rows(x)
    for n, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s >= 0:
            kv_fp4[s // bs, s % bs] = packed[n]
            kv_scale[s // bs, s % bs] = sc[n]
    return kv_fp4, kv_scale
