"""The fp8 row producer's quotient method, checked on the host.

The kernel does not divide in float32: it takes the row scale's reciprocal
once in float64 (a correctly rounded division) and rounds double(x) * rs to
float32 per element. The claim is that this equals the IEEE float32
quotient x / s wherever |x / s| >= 2^-10 (below that every e4m3 code is a
signed zero): a float32 quotient is never within 2^-49 (relative) of a
float32 rounding midpoint, and the double product is within 2^-52 of it.
numpy's float32 division is the IEEE one. The cases are random row values
at random scales, subnormal scales, and pairs built to land next to a
rounding midpoint, where a wrong method would round the other way.
"""
import numpy as np


def _method(x, s):
    rs = 1.0 / s.astype(np.float64)
    return (x.astype(np.float64) * rs).astype(np.float32)


def _check(x, s):
    x = np.asarray(x, np.float32)
    s = np.asarray(s, np.float32)
    with np.errstate(all="ignore"):
        ref = x / s
    got = _method(x, s)
    keep = np.abs(ref) >= np.float32(2.0 ** -10)
    bad = keep & (got.view(np.uint32) != ref.view(np.uint32))
    assert not bad.any(), (x[bad][:4], s[bad][:4], got[bad][:4], ref[bad][:4])
    return int(keep.sum())


def test_random_rows():
    rng = np.random.default_rng(11)
    n = 2_000_000
    amax = np.exp2(rng.uniform(-120, 120, n)).astype(np.float32)
    s = (amax / np.float32(448)).astype(np.float32)
    x = (rng.uniform(-1, 1, n) * amax).astype(np.float32)
    assert _check(x, s) > n // 2


def test_subnormal_scales():
    rng = np.random.default_rng(12)
    n = 500_000
    s = (rng.integers(1, 1 << 23, n).astype(np.uint32)).view(np.float32)  # every subnormal float32
    x = (rng.uniform(-448, 448, n) * s.astype(np.float64)).astype(np.float32)
    assert _check(x, s) > n // 2


def test_next_to_midpoints():
    """x = float32(M * s) for midpoints M between consecutive float32 numbers:
    the exact quotient x / s then lies within a few float32 ulps of M."""
    rng = np.random.default_rng(13)
    n = 2_000_000
    e = rng.integers(-10, 9, n)                                   # M in [2^-10, 2^9)
    mant = rng.integers(1 << 23, 1 << 24, n)                      # 24-bit significand
    m = (mant.astype(np.float64) + 0.5) * np.exp2(e - 23.0)       # the midpoint above it
    s = np.exp2(rng.uniform(-60, 60, n)).astype(np.float32)
    x = (m * s.astype(np.float64)).astype(np.float32)
    for dx in (-1, 0, 1):                                         # and the neighbouring x
        xx = (x.view(np.int32) + dx).view(np.float32)
        assert _check(xx, s) > n // 2
