"""Pins for oracle/formats.py against library codecs, golden tables and exact search."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import golden
import _exact
from oracle import formats as F


def test_e2m1_values_match_ocp_table():
    want = golden("e2m1_table.json")["values"]
    got = F.e2m1_value(np.arange(16))
    assert np.array_equal(got, np.array(want))
    assert np.array_equal(np.signbit(got), np.signbit(np.array(want)))


def test_e4m3_values_match_torch_codec():
    bytes_ = torch.arange(256, dtype=torch.uint8)
    ref = bytes_.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_value(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert F.e4m3_value(0x7E) == 448.0 and F.e4m3_value(0x01) == 2.0 ** -9


def test_e8m0_values_match_torch_codec():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = F.e8m0_value(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_int4_values_are_twos_complement():
    n = np.arange(16, dtype=np.uint8)
    ref = ((n << 4).astype(np.uint8).view(np.int8) >> 4).astype(np.float64)   # sign-extend via int8
    assert np.array_equal(F.int4_value(n), ref)
    assert np.array_equal(F.int4_encode(np.arange(-8, 8)), (np.arange(-8, 8) & 15).astype(np.uint8))


def _bf16_fp32_inputs(rng, n):
    bits = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # ties: low 16 bits exactly 0x8000, both parities of the kept part
    tie = (rng.integers(0, 2 ** 16, 2000).astype(np.uint32) << 16) | np.uint32(0x8000)
    tie = tie.view(np.float32)
    sub = (rng.integers(0, 2 ** 23, 2000).astype(np.uint32)).view(np.float32)    # subnormals
    big = np.array([3.3895314e38, 3.4e38, np.finfo(np.float32).max, -3.39e38], np.float32)
    return np.concatenate([x, tie[np.isfinite(tie)], sub, big])


def test_bf16_rounding_matches_torch_for_fp32_inputs():
    x = _bf16_fp32_inputs(np.random.default_rng(0), 200000)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.bf16_from_f64(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_rounding_is_nearest_even_for_fp64_inputs():
    rng = np.random.default_rng(1)
    y = rng.standard_normal(3000) * np.ldexp(1.0, rng.integers(-140, 120, 3000))
    # fp64 values within one fp64 ulp of a bf16 midpoint (where double rounding via fp32 would fail)
    mids = (F.bf16_value(rng.integers(0x0080, 0x7F00, 500).astype(np.uint16)) * (1 + 2.0 ** -8))
    y = np.concatenate([y, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf)])
    got = F.bf16_from_f64(y)
    for v, b in zip(y, got):
        b = int(b)
        target = Fraction(float(v))
        cands = [(c, _exact.bf16_value_exact(c)) for c in (b - 1, b, b + 1) if (c & 0x7F80) != 0x7F80]
        sign = 0x8000 if v < 0 else 0
        cands = [(c, val) for c, val in cands if (c & 0x8000) == sign or val == 0]
        assert _exact.nearest_even(target, cands) == b, (v, hex(b))


def test_bf16_overflow_and_signed_zero():
    big = float(np.ldexp(255.5, 120))          # exactly half way above the largest bf16
    assert F.bf16_from_f64(np.array([big]))[0] == 0x7F80
    assert F.bf16_from_f64(np.array([np.nextafter(big, 0)]))[0] == 0x7F7F
    assert F.bf16_from_f64(np.array([-0.0]))[0] == 0x8000
    assert F.bf16_from_f64(np.array([2.0 ** -134]))[0] == 0x0000     # tie with 0 -> even
    assert F.bf16_from_f64(np.array([3 * 2.0 ** -134]))[0] == 0x0002  # tie 1|2 -> even


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(2)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = list(rng.uniform(-8, 8, 400)) + mids + [-m for m in mids] + \
        [0.0, -0.0, 6.0, 6.5, 100.0, -7.9, 1e-30, -1e-30, 0.2499999, 0.2500001]
    for unit in (1.0, 0.5, 2.0 ** -20, 2.0 ** 7):
        xs = np.array(vals) * unit
        got = F.e2m1_encode(xs, unit)
        for x, g in zip(xs, got):
            assert g == _exact.e2m1_code(float(x), unit), (x, unit, g)


def test_e2m1_encode_non_power_of_two_unit():
    rng = np.random.default_rng(3)
    unit = float(F.e4m3_value(0x5D)) * float(np.float32(0.0123))   # E4M3 value times an fp32 value
    xs = np.concatenate([rng.uniform(-7, 7, 300) * unit, np.array([0.75, 1.75, 3.5, 5.0]) * unit])
    got = F.e2m1_encode(xs, unit)
    for x, g in zip(xs, got):
        assert g == _exact.e2m1_code(float(x), unit)


def test_e4m3_encode_matches_torch_for_in_range_values():
    rng = np.random.default_rng(4)
    x = np.abs(rng.standard_normal(20000) * np.ldexp(1.0, rng.integers(-14, 9, 20000))).astype(np.float32)
    x = np.concatenate([x, F.E4M3_MIDPOINTS.astype(np.float32), np.float32(F.E4M3_GRID)])
    x = x[x <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode_ratio(x.astype(np.float64), 1.0)
    assert np.array_equal(got, ref)


def test_e4m3_encode_ratio_brute_force_and_saturation():
    rng = np.random.default_rng(5)
    den = 6.0 * float(np.float32(0.000733))
    nums = list(np.abs(rng.standard_normal(300)) * den * np.ldexp(1.0, rng.integers(-12, 10, 300)))
    nums += [float(F.E4M3_MIDPOINTS[j] * den) for j in range(0, 126, 5)]
    got = F.e4m3_encode_ratio(np.array(nums), den)
    for n, g in zip(nums, got):
        assert g == _exact.e4m3_code(Fraction(n) / Fraction(den)), (n, g)
    assert F.e4m3_encode_ratio(np.array([1e6, 464.0, 463.9]), 1.0).tolist() == [0x7E, 0x7E, 0x7E]
    assert F.e4m3_encode_ratio(np.array([2.0 ** -10, 2.0 ** -10 * 1.0001]), 1.0).tolist() == [0, 1]
