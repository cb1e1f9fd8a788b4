"""Pins of the oracle's INT4 G=64 format (BF16 block scales): the paper's
packed deployment format (Appendix I), with Section 3's symmetric scale
Delta = max|x| / 7 on the INT4 grid and Section 4.2's BF16 admissible set.

The scale is checked against exact rational rounding to BF16 (every
candidate BF16 value near amax / 7 compared with fractions.Fraction), the
elements against a brute-force search of the 16 codes, and the whole layer
against an exact rational evaluation."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int4g64_blocks.json")


def bf16_candidates():
    """Every finite non-negative BF16 value with its bit pattern."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    return bits, vals


BITS, VALS = bf16_candidates()


def exact_bf16_of_quotient(num, den):
    """Nearest BF16 to the rational num/den (ties to the even pattern), by
    comparing exact distances to the two neighbouring BF16 values."""
    q = Fraction(num) / Fraction(den)
    i = int(np.searchsorted(VALS, float(q)))
    best = None
    for j in range(max(0, i - 2), min(len(VALS), i + 3)):
        d = abs(Fraction(VALS[j]) - q)
        key = (d, int(BITS[j]) & 1)
        if best is None or key < best[0]:
            best = (key, int(BITS[j]))
    return best[1]


def brute_code(x, delta):
    """argmin over the 16 INT4 codes of |x - code * delta| (exact), ties to the even code."""
    if delta == 0:
        return 0
    xs = Fraction(x)
    d = Fraction(delta)
    return min(range(-8, 8), key=lambda k: (abs(xs - k * d), k & 1))


def quantize_one_block(x):
    codes, scales, _ = oracle.quantize_rows(np.asarray(x, np.float32)[None, :], "int4g64")
    return F.int4_value(codes[0]).astype(int), int(scales[0, 0])


def test_block_size_and_scale_storage():
    assert oracle.BLOCK["int4g64"] == 64
    codes, scales, t = oracle.quantize_rows(np.ones((3, 256), np.float32), "int4g64")
    assert scales.dtype == np.uint16 and scales.shape == (3, 4) and t is None
    # Table 12: G=64 BF16 scales cost as many bytes as G=32 E8M0 scales
    _, mx, _ = oracle.quantize_rows(np.ones((3, 256), np.float32), "mxfp4")
    assert scales.nbytes == mx.nbytes


def test_golden_blocks():
    with open(GOLDEN) as f:
        g = json.load(f)
    for blk in g["blocks"]:
        x = np.zeros(64, np.float32)
        for k, v in blk["x"].items():
            x[int(k)] = v
        codes, bits = quantize_one_block(x)
        assert bits == blk["delta_bits"], blk["name"]
        want = np.zeros(64, int)
        for k, v in blk["codes"].items():
            want[int(k)] = v
        assert np.array_equal(codes, want), blk["name"]


def test_scale_is_exact_rounding_of_amax_over_7():
    rng = np.random.default_rng(0)
    amax = np.ldexp(rng.uniform(0.5, 1.0, 300), rng.integers(-150, 127, 300)).astype(np.float32)
    # exact ties: 7 * (BF16 midpoints) that fp32 holds exactly
    mids = np.float32(7.0) * (np.float32(1.0) + np.float32(2.0 ** -8) * np.arange(1, 256, 2, dtype=np.float32))
    special = np.array([2.0 ** -149, 2.0 ** -140, 7 * 2.0 ** -133, 3.4e38, 7.0, 1.0], np.float32)
    for a in np.concatenate([amax, mids.astype(np.float32), special]):
        a = np.float32(a)
        if a == 0:
            continue
        x = np.zeros(64, np.float32)
        x[5] = a
        _, bits = quantize_one_block(x)
        assert bits == exact_bf16_of_quotient(float(a), 7), float(a)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_elements_match_brute_force(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(64) * np.exp(rng.normal(0, 2))).astype(np.float32)
    if seed == 2:
        x[:8] = 0.0                          # zeros
    if seed == 3:                            # values that land on half-integers of Delta
        codes, bits = quantize_one_block(x)
        delta = float(F.bf16_value(np.uint16(bits)))
        x[:16] = (np.arange(-8, 8) + 0.5).astype(np.float32) * np.float32(delta)
        x[16] = np.float32(7 * delta)
    codes, bits = quantize_one_block(x)
    delta = float(F.bf16_value(np.uint16(bits)))
    assert bits == exact_bf16_of_quotient(float(np.max(np.abs(x))), 7)
    for v, c in zip(x, codes):
        assert c == brute_code(float(v), delta), (float(v), delta)


def test_zero_block_and_underflowing_scale():
    codes, bits = quantize_one_block(np.zeros(64, np.float32))
    assert bits == 0 and not codes.any()
    # amax / 7 below half the smallest BF16 subnormal (2^-134) rounds to 0
    x = np.zeros(64, np.float32)
    x[3] = np.float32(2.0 ** -149)
    codes, bits = quantize_one_block(x)
    assert bits == 0 and not codes.any()


def test_nonfinite_convention():
    x = np.ones(64, np.float32)
    x[7] = np.inf
    codes, bits = quantize_one_block(x)
    assert bits == 0x7FC0 and not codes.any()


def test_round_trip_of_representable_blocks():
    rng = np.random.default_rng(4)
    for _ in range(20):
        q = rng.integers(-7, 8, 64)
        q[rng.integers(0, 64)] = rng.choice([-7, 7])
        delta_bits = np.uint16(rng.integers(0x3000, 0x4F00))
        delta = F.bf16_value(delta_bits)
        x = (q * delta).astype(np.float32)
        assert np.array_equal(x.astype(np.float64), q * delta)      # exactly representable
        codes, bits = quantize_one_block(x)
        assert bits == delta_bits and np.array_equal(codes, q)


def test_power_of_two_scaling_and_negation():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    c0, s0, _ = oracle.quantize_rows(x, "int4g64")
    c1, s1, _ = oracle.quantize_rows(np.ldexp(x, 5).astype(np.float32), "int4g64")
    assert np.array_equal(c0, c1)
    assert np.array_equal(F.bf16_value(s1), np.ldexp(F.bf16_value(s0), 5))
    c2, s2, _ = oracle.quantize_rows(-x, "int4g64")
    assert np.array_equal(s2, s0)
    assert np.array_equal(F.int4_value(c2), -F.int4_value(c0))


def test_dequantize_is_code_times_scale():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 192)).astype(np.float32)
    codes, scales, _ = oracle.quantize_rows(x, "int4g64")
    deq = oracle.dequantize(oracle.pack_nibbles(codes), scales, "int4g64")
    for i in range(3):
        for k in range(0, 192, 17):
            assert deq[i, k] == F.int4_value(codes[i, k]) * F.bf16_value(scales[i, k // 64])


def test_layer_matches_exact_rational_evaluation():
    """Y = BF16(r[n] * sum_b Delta_a Delta_w sum_k qa qw), evaluated with Fractions."""
    rng = np.random.default_rng(7)
    M, N, K = 3, 4, 128
    x = rng.standard_normal((M, K)).astype(np.float32)
    c = F.bf16_value(F.bf16_from_f64(np.exp(rng.normal(0, 0.5, K)))).astype(np.float32)
    r = F.bf16_value(F.bf16_from_f64(np.exp(rng.normal(0, 0.5, N)))).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    wc, ws, tw = oracle.quantize_weight(w, "int4g64")
    ac, as_, ta, bits, y = oracle.layer(x, c, wc, ws, tw, r, "int4g64")
    qa, qw = F.int4_value(oracle.unpack_nibbles(ac)), F.int4_value(oracle.unpack_nibbles(wc))
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for b in range(K // 64):
                dot = sum(int(qa[m, k]) * int(qw[n, k]) for k in range(64 * b, 64 * b + 64))
                tot += Fraction(float(F.bf16_value(as_[m, b]))) * Fraction(float(F.bf16_value(ws[n, b]))) * dot
            exact = tot * Fraction(float(r[n]))
            assert Fraction(y[m, n]) == exact
            assert bits[m, n] == F.bf16_from_f64(np.float64(exact))
    # the activation really is the fp32 product X * c, quantized
    ac2, as2, _ = oracle.quantize_act((x.astype(np.float64) * c).astype(np.float32), np.ones(K, np.float32), "int4g64")
    assert np.array_equal(ac2, ac) and np.array_equal(as2, as_)
