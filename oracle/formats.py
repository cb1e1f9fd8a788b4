"""Number formats of the block-scaled 4-bit path: plain CPU definitions.

TEST INFRASTRUCTURE ONLY.  This package is the oracle: a slow, obviously
correct fp64 restatement of what the packed W4A4 path computes.  Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
it; the product path never does.

Formats (DualQuant, Section 3 "Quantization preliminaries": MXFP4 and
MXINT4 use blocks of 32 with a shared power-of-two E8M0 scale, NVFP4 uses
blocks of 16 with an FP8 UE4M3 scale; the element grids are the integer grid
for INT formats and the exponent-mantissa grid for FP formats; Appendix G.2
adds the 8-bit MXFP8 and MXINT8, blocks of 32 with E8M0 scales).  The bit
layouts are the OCP Microscaling / OCP FP8 definitions that section cites:

* E2M1 : sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
         0, 0.5, 1, 1.5, 2, 3, 4, 6; no inf/NaN.
* E4M3 : FP8 "FN" variant, bias 7, subnormals m * 2^-9, max 448,
         0x7F / 0xFF are NaN, no infinities.
* E8M0 : unsigned exponent, value 2^(b-127), 0xFF is NaN.
* INT4 : two's complement nibble, -8..7.
* INT8 : two's complement byte, -128..127 (the MXINT8 elements, Appendix
         G.2's 8-bit variants).
* BF16 : IEEE-style 1/8/7; results are rounded once, from fp64, to nearest
         with ties to even.

All encoders decide by exact comparisons against midpoints between
neighbouring grid values ("round to the nearest point of the grid", Section
3), ties going to the even code, magnitudes beyond the grid clipping to its
largest value.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------- E2M1 ----


def e2m1_value(code):
    """Decode 4-bit E2M1 codes (array of ints 0..15) to float64."""
    code = np.asarray(code).astype(np.int64)
    sign = np.where(code & 8, -1.0, 1.0)
    e = (code >> 1) & 3
    m = code & 1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, e - 1))
    return sign * mag


E2M1_GRID = e2m1_value(np.arange(8))              # 0, .5, 1, 1.5, 2, 3, 4, 6
E2M1_MIDPOINTS = (E2M1_GRID[:-1] + E2M1_GRID[1:]) / 2.0


def _rne_index(a, thresholds):
    """Index of the nearest grid point for magnitudes a.

    thresholds[..., j] is the exact midpoint between grid points j and j+1,
    in the units of a, broadcastable against a[..., None].  The index is the
    number of midpoints strictly below a, plus one where a sits exactly on a
    midpoint whose upper neighbour j+1 is the even code (ties to even).
    Magnitudes beyond the last midpoint land on the last grid point (clip).
    """
    a = np.asarray(a, np.float64)[..., None]
    thresholds = np.asarray(thresholds, np.float64)
    upper_is_even = (np.arange(1, thresholds.shape[-1] + 1) % 2) == 0
    above = (a > thresholds).sum(axis=-1)
    tie_up = ((a == thresholds) & upper_is_even).sum(axis=-1)
    return above + tie_up


def e2m1_encode(x, unit):
    """E2M1 code of x / unit, round to nearest even, saturating at +-6.

    x    : fp64 array (exact values); the sign bit of x becomes the code's
           sign bit, so negative inputs that round to zero give 0x8.
    unit : positive fp64, broadcastable to x, such that every
           midpoint * unit is exact in fp64 (true for power-of-two units and
           for products of an E4M3 value with an fp32 value).
    """
    x = np.asarray(x, np.float64)
    unit = np.asarray(unit, np.float64)
    thr = E2M1_MIDPOINTS * unit[..., None]
    idx = _rne_index(np.abs(x), thr)
    sign = np.signbit(x).astype(np.int64) << 3
    return (idx | sign).astype(np.uint8)


# ----------------------------------------------------------------- E4M3 ----


def e4m3_value(byte):
    """Decode FP8 E4M3 (FN) bytes to float64; 0x7F/0xFF give NaN."""
    b = np.asarray(byte).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


E4M3_GRID = e4m3_value(np.arange(0x7F))          # codes 0x00..0x7E, 0 .. 448
E4M3_MIDPOINTS = (E4M3_GRID[:-1] + E4M3_GRID[1:]) / 2.0
E4M3_MAX = 448.0


def e4m3_encode_ratio(num, den):
    """UE4M3 code of the exact real num/den (num >= 0, den > 0), RNE, saturating.

    Decided by comparing num with midpoint * den, exact in fp64 whenever den
    has at most 48 significant bits (midpoints have at most 5).
    """
    num = np.asarray(num, np.float64)
    den = np.asarray(den, np.float64)
    thr = E4M3_MIDPOINTS * den[..., None]
    return _rne_index(num, thr).astype(np.uint8)


def e4m3_encode(x, unit):
    """Signed E4M3 code of x / unit, round to nearest even, saturating at +-448.

    x    : fp64 array (exact values); the sign bit of x becomes the code's
           bit 7, so negative inputs that round to zero give 0x80.
    unit : positive fp64 power of two, broadcastable to x (every midpoint *
           unit is then exact in fp64).
    """
    x = np.asarray(x, np.float64)
    unit = np.asarray(unit, np.float64)
    idx = e4m3_encode_ratio(np.abs(x), unit)
    sign = np.signbit(x).astype(np.int64) << 7
    return (idx.astype(np.int64) | sign).astype(np.uint8)


# ----------------------------------------------------------------- E8M0 ----


def e8m0_value(byte):
    b = np.asarray(byte).astype(np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


# ----------------------------------------------------------------- INT4 ----


def int4_value(nibble):
    n = np.asarray(nibble).astype(np.int64) & 15
    return np.where(n >= 8, n - 16, n).astype(np.float64)


def int4_encode(v):
    """Two's complement nibble of integer-valued v in [-8, 7]."""
    return (np.asarray(v).astype(np.int64) & 15).astype(np.uint8)


# ----------------------------------------------------------------- INT8 ----


def int8_value(byte):
    b = np.asarray(byte).astype(np.int64) & 255
    return np.where(b >= 128, b - 256, b).astype(np.float64)


def int8_encode(v):
    """Two's complement byte of integer-valued v in [-128, 127]."""
    return (np.asarray(v).astype(np.int64) & 255).astype(np.uint8)


# ----------------------------------------------------------------- BF16 ----

BF16_MAX = float(np.ldexp(255.0, 120))            # (2 - 2^-7) * 2^127


def bf16_from_f64(y):
    """Round fp64 values once to bfloat16 (nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Normal bf16 values carry 8
    significant bits; below 2^-126 the spacing is fixed at 2^-133.  Values
    that round beyond the largest finite bf16 become infinities.
    """
    y = np.asarray(y, np.float64)
    mag = np.abs(y)
    _, E = np.frexp(mag)                           # mag = f * 2^E, f in [0.5, 1)
    qexp = np.maximum(E - 8, -133)                  # exponent of one unit in the last place
    n = np.rint(np.ldexp(mag, -qexp))               # exact scaling, then RNE to integer
    rounded = np.ldexp(n, qexp)
    rounded = np.where(rounded > BF16_MAX, np.inf, rounded)
    val = np.copysign(rounded, y)
    bits = (val.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(y), np.uint16(0x7FC0), bits)


def bf16_value(bits):
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
