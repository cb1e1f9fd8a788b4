"""Exact rational helpers for pinning the oracle (fractions.Fraction).

Written independently of oracle/: values come from the golden E2M1 table and
from first-principles bit decoding, nearest-point searches are exhaustive.
"""
import math
from fractions import Fraction

from conftest import golden

E2M1 = [Fraction(v) for v in golden("e2m1_table.json")["values"][:8]]   # magnitudes of codes 0..7


def e4m3_exact(byte):
    """Exact value of a non-negative finite E4M3 byte (0x00..0x7E)."""
    e, m = (byte >> 3) & 15, byte & 7
    if e == 0:
        return Fraction(m, 512)
    return Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


def nearest_even(target, candidates):
    """Code of the candidate nearest to target; equal distances -> even code.

    candidates: list of (code, exact value).
    """
    best = None
    for code, val in candidates:
        d = abs(target - val)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0 and best[1] % 2 == 1):
            best = (d, code)
    return best[1]


def e2m1_code(x, unit):
    """E2M1 code of the exact real x/unit: nearest of the 8 magnitudes, even on ties, sign of x."""
    neg = math.copysign(1.0, float(x)) < 0
    mag = nearest_even(abs(Fraction(x)) / Fraction(unit), list(enumerate(E2M1)))
    return mag | (8 if neg else 0)


def e4m3_code(u):
    """UE4M3 byte nearest to the exact real u >= 0 (even on ties, saturating at 448)."""
    return nearest_even(Fraction(u), [(b, e4m3_exact(b)) for b in range(0x7F)])


def bf16_value_exact(bits):
    s = -1 if bits & 0x8000 else 1
    e, m = (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0:
        return s * Fraction(m) * Fraction(2) ** -133
    return s * Fraction(128 + m) * Fraction(2) ** (e - 134)
