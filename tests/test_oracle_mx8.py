"""Pins for the oracle's 8-bit MX formats (DualQuant Appendix G.2, Table 9:
MXFP8 and MXINT8 with G = 32 and E8M0 scales).

Independent of oracle/: exhaustive nearest-point searches over every finite
E4M3 code and every int8 value in exact rational arithmetic, torch's own
float8_e4m3fn codec, the shared-exponent rule at its binade edges, round
trips, power-of-two scaling, negation, hand-worked golden blocks and an
exact rational evaluation of a small layer."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import golden
import _exact
import oracle
from oracle import formats as F
from oracle.quant import quantize_rows, quantize_act, dequantize, pack_codes

E4M3_POS = [(b, _exact.e4m3_exact(b)) for b in range(0x7F)]       # 0 .. 448


def e4m3_signed_code(v, unit):
    """Brute force: nearest of the 127 magnitudes (even code on ties, 448 at
    most), the sign bit of v on top (so -0 is 0x80)."""
    neg = math.copysign(1.0, float(v)) < 0
    mag = _exact.nearest_even(abs(Fraction(float(v))) / unit, E4M3_POS)
    return mag | (0x80 if neg else 0)


def int8_code(v, unit):
    q = Fraction(float(v)) / unit
    best = min(range(-128, 128), key=lambda n: (abs(q - n), n % 2))
    return best & 255


def floor_log2(a):
    f = Fraction(float(a))
    e = 0
    while Fraction(2) ** e > f:
        e -= 1
    while Fraction(2) ** (e + 1) <= f:
        e += 1
    return e


def random_blocks(rng, R, K):
    x = rng.standard_normal((R, K)) * np.ldexp(1.0, rng.integers(-30, 30, (R, 1)))
    x[0, :8] = [17.0, 19.0, 1.0625, -3.0, 448.0, 464.0, 0.0, -0.0]       # E4M3 ties and saturation at e = 0
    x[1, :8] = [127.5, -127.5, 2.5, 3.5, -0.5, 64.0, 100.25, 0.0]       # int8 ties at e = 0
    x[2, 32:36] = [2.0 ** -140, -2.0 ** -149, 0.0, -0.0]               # subnormals and zeros
    return x.astype(np.float32)


@pytest.mark.parametrize("fmt,emax", [("mxfp8", 8), ("mxint8", 6)])
def test_mx8_brute_force(fmt, emax):
    rng = np.random.default_rng(11)
    x = random_blocks(rng, 6, 128)
    codes, scales, t = quantize_rows(x, fmt)
    assert t is None and codes.shape == x.shape
    for m in range(x.shape[0]):
        for b in range(4):
            blk = x[m, 32 * b:32 * b + 32]
            amax = float(np.max(np.abs(blk)))
            e = -127 if amax == 0 else max(-127, min(127, floor_log2(amax) - emax))
            assert scales[m, b] == e + 127, (m, b)
            unit = Fraction(2) ** e
            for i, v in enumerate(blk):
                want = e4m3_signed_code(v, unit) if fmt == "mxfp8" else int8_code(v, unit)
                assert codes[m, 32 * b + i] == want, (fmt, m, b, i, v)


def test_mxfp8_elements_agree_with_torch_float8():
    """In range (|v| < 464, where no saturation applies), the element code is
    torch's own round-to-nearest-even float8_e4m3fn encoding of x~ * 2^-e."""
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((64, 256)) * np.ldexp(1.0, rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    codes, scales, _ = quantize_rows(x, "mxfp8")
    e = scales.astype(np.int64) - 127
    v = np.ldexp(x.astype(np.float64).reshape(64, 8, 32), -e[..., None]).reshape(64, 256)
    ok = np.abs(v) < 464
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert ok.mean() > 0.99
    assert np.array_equal(codes[ok], ref[ok])


@pytest.mark.parametrize("k", [-40, -3, 0, 7, 50])
def test_mx8_shared_exponent_rule(k):
    def one(fmt, amax):
        x = np.zeros((1, 32), np.float32)
        x[0, 5] = amax
        codes, scales, _ = quantize_rows(x, fmt)
        return int(scales[0, 0]), int(codes[0, 5])
    # MXFP8: 256 * 2^k is E4M3 256 (0x78) at byte 127 + k; just below 512 * 2^k
    # keeps the byte and saturates to 448 (0x7E); 512 * 2^k moves the byte up
    assert one("mxfp8", math.ldexp(256.0, k)) == (127 + k, 0x78)
    assert one("mxfp8", math.ldexp(512.0 * (1 - 2 ** -24), k)) == (127 + k, 0x7E)
    assert one("mxfp8", math.ldexp(512.0, k)) == (128 + k, 0x78)
    assert one("mxfp8", -math.ldexp(448.0, k)) == (127 + k, 0xFE)
    # MXINT8: 64 * 2^k -> code 64; just below 128 * 2^k -> 127 (clipped);
    # 128 * 2^k -> byte up, code 64
    assert one("mxint8", math.ldexp(64.0, k)) == (127 + k, 64)
    assert one("mxint8", math.ldexp(128.0 * (1 - 2 ** -24), k)) == (127 + k, 127)
    assert one("mxint8", math.ldexp(128.0, k)) == (128 + k, 64)
    assert one("mxint8", -math.ldexp(127.5, k)) == (127 + k, 0x80)      # -128 stays representable


@pytest.mark.parametrize("fmt", ["mxfp8", "mxint8"])
def test_mx8_round_trip_of_representable_blocks(fmt):
    """Blocks built from codes and a scale, whose largest element lies in the
    top binade of the element grid, quantize back to those codes and scale."""
    rng = np.random.default_rng(13)
    sbytes = list(range(70, 190, 7))
    rows, want = [], []
    for s in sbytes:
        if fmt == "mxfp8":
            c = rng.integers(0, 256, 32)
            c = np.where((c & 0x7F) == 0x7F, c - 1, c)                # no NaN codes
            c[rng.integers(32)] = rng.choice([0x78, 0x7E, 0xFB])       # |value| in [256, 448]
            vals = F.e4m3_value(c) * 2.0 ** (s - 127)
        else:
            c = rng.integers(-127, 128, 32)
            c[rng.integers(32)] = rng.choice([64, 127, -100])
            vals = c * 2.0 ** (s - 127)
            c = c & 255
        rows.append(vals)
        want.append(c)
    x = np.array(rows, np.float32)
    assert np.array_equal(x.astype(np.float64), np.array(rows))
    codes, scales, _ = quantize_rows(x, fmt)
    assert scales[:, 0].tolist() == sbytes
    assert np.array_equal(codes, np.array(want, np.uint8))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxint8"])
def test_mx8_scaling_and_negation(fmt):
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((8, 128)) * 3).astype(np.float32)
    x[0, :4] = [127.5, 7.0, 0.0, 1.0]
    c0, s0, _ = quantize_rows(x, fmt)
    for j in (-11, 2, 30):
        c1, s1, _ = quantize_rows(x * np.float32(2.0 ** j), fmt)
        assert np.array_equal(c0, c1) and np.array_equal(s1.astype(int), s0.astype(int) + j)
    cn, sn, _ = quantize_rows(-x, fmt)
    assert np.array_equal(sn, s0)
    if fmt == "mxfp8":
        assert np.array_equal(cn, c0 ^ 0x80)
    else:
        v0, v1 = F.int8_value(c0), F.int8_value(cn)
        clipped = (v0 == 127) & (v1 == -128)
        assert np.array_equal(v1[~clipped], -v0[~clipped]) and clipped.any()


@pytest.mark.parametrize("fmt", ["mxfp8", "mxint8"])
def test_mx8_golden_block(fmt):
    g = golden(f"{fmt}_block.json")
    x = np.array([g["x"]], np.float32)
    assert np.array_equal(F.bf16_value(F.bf16_from_f64(x)), x.astype(np.float64))
    codes, scales, _ = quantize_act(x, np.ones(32, np.float32), fmt)
    assert codes[0].tolist() == g["codes"]
    assert scales[0].tolist() == [g["scale"]]


def test_mx8_nonfinite_convention():
    x = np.ones((1, 64), np.float32)
    x[0, 3] = np.inf
    for fmt in ("mxfp8", "mxint8"):
        codes, scales, _ = quantize_rows(x, fmt)
        assert scales[0, 0] == 255 and (codes[0, :32] == 0).all()


@pytest.mark.parametrize("fmt", ["mxfp8", "mxint8"])
def test_mx8_layer_matches_exact_rational_evaluation(fmt):
    """Y = BF16(r[n] * sum_k a^ w^) against a Fraction evaluation built from
    first-principles decoding of the codes and scales."""
    rng = np.random.default_rng(15)
    M, N, K = 3, 5, 96
    x = F.bf16_value(F.bf16_from_f64(rng.standard_normal((M, K)) * 4)).astype(np.float32)
    c = np.ldexp(1.0, rng.integers(-2, 3, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    r = np.ldexp(1.0, rng.integers(-3, 3, N)).astype(np.float32)
    wc, ws, tw = oracle.quantize_weight(w, fmt)
    ac, as_, ta, bits, y = oracle.layer(x, c, wc, ws, tw, r, fmt)

    def val(code):
        if fmt == "mxint8":
            return Fraction(int(code) - 256 if code >= 128 else int(code))
        s = -1 if code & 0x80 else 1
        return s * _exact.e4m3_exact(int(code) & 0x7F)

    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for k in range(K):
                sa = Fraction(2) ** (int(as_[m, k // 32]) - 127)
                sw = Fraction(2) ** (int(ws[n, k // 32]) - 127)
                tot += val(ac[m, k]) * sa * val(wc[n, k]) * sw
            tot *= Fraction(float(r[n]))
            assert Fraction(float(y[m, n])) == tot
            want = F.bf16_from_f64(np.array([float(tot)]))[0]
            assert bits[m, n] == want


def test_mx8_codes_are_one_byte_per_element():
    """Small integers are exact in both grids: -7..7 in MXFP8 (amax 7 -> e = -6,
    7 * 64 = 448), -63..63 in MXINT8 (amax 63 -> e = -1, 63 * 2 = 126)."""
    for fmt, top in (("mxfp8", 7), ("mxint8", 63)):
        x = (np.arange(64) % (2 * top + 1) - top).astype(np.float32).reshape(1, 64)
        x[0, 0] = x[0, 32] = top
        codes, scales, _ = quantize_act(x, np.ones(64, np.float32), fmt)
        assert codes.shape == (1, 64) and scales.shape == (1, 2)
        assert np.array_equal(pack_codes(codes, fmt), codes)
        deq = dequantize(codes, scales, fmt)
        assert np.array_equal(deq, x.astype(np.float64))
