"""Number-format decoders of the oracle, each written from its closed form.

* bf16: the upper 16 bits of an IEEE binary32.
* OCP e4m3 ("e4m3fn"): sign, 4 exponent bits (bias 7), 3 mantissa bits;
  exponent 0 is subnormal, S.1111.111 is NaN, no infinities.  The pages note
  that MI325X and newer use this OCP encoding while gfx942 uses the fnuz one
  (page "DeepSeek V4 Flash on a single AMD MI300X", section "Why MI300X" and
  the "FP8 format" correctness fix).
* E2M1 (mxfp4 element): sign, 2 exponent bits (bias 1), 1 mantissa bit; the
  gather decodes it arithmetically (page "xkernels #28 -- DeepSeek-V4 serving
  support", comment shipping mxfp4_paged_gather).
* E8M0 (mxfp4 group scale): 2**(b-127), with byte 0xFF read as 0 (same comment).
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 storage bits (uint16) -> exact float64 value."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_to_f64(code) -> np.ndarray:
    """OCP e4m3 byte -> exact float64 value (NaN for 0x7F / 0xFF)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int64))
    subnormal = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 0xF) & ((c & 7) == 7), np.nan, v)


def e2m1_to_f64(nibble) -> np.ndarray:
    """E2M1 nibble (0..15) -> exact float64 value; codes give 0,.5,1,1.5,2,3,4,6."""
    c = np.asarray(nibble, dtype=np.int64) & 0xF
    sign = np.where(c >> 3, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    normal = (1.0 + m / 2.0) * np.ldexp(1.0, (e - 1).astype(np.int64))
    subnormal = m / 2.0
    return sign * np.where(e == 0, subnormal, normal)


def e8m0_to_f64(byte) -> np.ndarray:
    """E8M0 scale byte -> 2**(b-127); 0xFF -> 0 (the gather's stated rule)."""
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 0xFF, 0.0, np.ldexp(1.0, b - 127))


def f64_to_bf16_bits(x) -> np.ndarray:
    """float64 -> bf16 bits, round to nearest even, gradual underflow, overflow to inf.

    bf16 keeps 8 significant bits with binary32's exponent range, so the
    quantum of a value in [2**e, 2**(e+1)) is 2**(e-7), never below the
    subnormal quantum 2**-133.
    """
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    _, e = np.frexp(mag)                      # mag = f * 2**e, f in [0.5, 1)
    quantum_exp = np.maximum(e - 1, -126) - 7
    r = np.ldexp(np.rint(np.ldexp(mag, -quantum_exp)), quantum_exp)  # rint = ties-to-even
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    r = np.where(np.isnan(x), np.nan, r)
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    sign = np.where(np.signbit(x), np.uint16(0x8000), np.uint16(0))
    return (bits | sign).astype(np.uint16)
