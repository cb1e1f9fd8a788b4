"""Pins for oracle/quant.py: hand-worked blocks, the shared-exponent rule,
round trips, invariances, exact brute force and sign preservation."""
import math
from fractions import Fraction

import numpy as np
import pytest

from conftest import golden
import _exact
import oracle
from oracle import formats as F
from oracle.quant import quantize_rows, quantize_act, pack_nibbles, unpack_nibbles, dequantize, rescale, nv_tensor_scale


def _bf16_exact(a):
    a = np.asarray(a, np.float32)
    assert np.array_equal(F.bf16_value(F.bf16_from_f64(a)), a.astype(np.float64))
    return a


@pytest.mark.parametrize("case", [0, 1])
def test_golden_mxfp4_block(case):
    g = golden("mxfp4_block.json")
    cs = g["cases"][case]
    x = _bf16_exact(np.array([g["x"]], np.float32))
    codes, scales, t = quantize_act(x, np.full(32, cs["c"], np.float32), "mxfp4")
    assert codes[0].tolist() == g["packed"]
    assert scales[0].tolist() == [cs["scale"]]
    assert t is None


def test_golden_mxint4_block():
    g = golden("mxint4_block.json")
    x = _bf16_exact([g["x"]])
    codes, scales, _ = quantize_act(x, np.ones(32, np.float32), "mxint4")
    assert unpack_nibbles(codes)[0].tolist() == g["codes"]
    assert scales[0].tolist() == [g["scale"]]


def test_golden_nvfp4_blocks():
    g = golden("nvfp4_blocks.json")
    x = _bf16_exact([g["x"]])
    codes, scales, t = quantize_act(x, np.ones(32, np.float32), "nvfp4")
    assert t == np.float32(g["t"])
    assert scales[0].tolist() == g["scales"]
    assert unpack_nibbles(codes)[0].tolist() == g["codes"]


@pytest.mark.parametrize("k", [-20, -3, 0, 5, 60])
def test_mx_shared_exponent_rule(k):
    """amax = 4*2^k -> byte 127+k (element 4.0); just below 8*2^k -> same byte,
    element saturates to 6; exactly 8*2^k -> byte 128+k."""
    def one(amax):
        x = np.zeros((1, 32), np.float32)
        x[0, 3] = amax
        codes, scales, _ = quantize_rows(x, "mxfp4")
        return int(scales[0, 0]), int(codes[0, 3])
    assert one(np.float32(math.ldexp(4.0, k))) == (127 + k, 0x6)
    assert one(np.float32(math.ldexp(8.0 * (1 - 2 ** -24), k))) == (127 + k, 0x7)
    assert one(np.float32(math.ldexp(8.0, k))) == (128 + k, 0x6)
    assert one(np.float32(math.ldexp(-6.0, k))) == (127 + k, 0xF)


def test_mxint4_shared_exponent_rule():
    def one(amax):
        x = np.zeros((1, 32), np.float32)
        x[0, 0] = amax
        codes, scales, _ = quantize_rows(x, "mxint4")
        return int(scales[0, 0]), int(codes[0, 0])
    assert one(4.0) == (127, 4)
    assert one(7.5) == (127, 7)          # rounds to 8, clipped to 7
    assert one(-7.5) == (127, 8)         # -8 stays representable
    assert one(7.49) == (127, 7)
    assert one(8.0) == (128, 4)
    assert one(0.375) == (127 - 4, 6)    # floor(log2 .375) = -2 -> e = -4, .375*16 = 6


def test_mx_scale_clamps_and_zero_block():
    x = np.zeros((1, 96), np.float32)
    x[0, 0] = np.float32(2.0 ** -149)                 # smallest subnormal
    x[0, 32] = np.finfo(np.float32).max
    codes, scales, _ = quantize_rows(x, "mxfp4")
    assert scales[0].tolist() == [0, 127 + 125, 0]    # clamp at -127; floor(log2 max) = 127
    assert codes[0, 0] == 0 and codes[0, 32] == 0x7   # 2^-149 * 2^127 = 2^-22 -> 0; max -> 6
    assert (codes[0, 64:] == 0).all()


def test_mx_nonfinite_convention():
    x = np.ones((2, 64), np.float32)
    x[0, 5] = np.inf
    x[1, 40] = np.nan
    for fmt in ("mxfp4", "mxint4"):
        codes, scales, _ = quantize_rows(x, fmt)
        assert scales[:, 0].tolist() == [255, 125] and scales[:, 1].tolist() == [125, 255]
        assert (codes[0, :32] == 0).all() and (codes[1, 32:] == 0).all()


def test_nv_block_at_tensor_amax_gets_largest_scale():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    codes, scales, t = quantize_rows(x, "nvfp4")
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert scales[i[0], i[1] // 16] == 0x7E
    assert codes[i] & 7 == 7                              # the amax element is +-6


def test_nv_tensor_scale_is_correctly_rounded_quotient():
    rng = np.random.default_rng(1)
    for _ in range(200):
        a = np.float32(abs(rng.standard_normal()) * 2.0 ** rng.integers(-100, 100))
        t = nv_tensor_scale(np.array([[a, -a / 2]], np.float32))
        exact = Fraction(float(a)) / 2688
        for nb in (np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(np.inf))):
            assert abs(Fraction(float(t)) - exact) <= abs(Fraction(float(nb)) - exact)
    assert nv_tensor_scale(np.zeros((2, 16), np.float32)) == 1.0


def test_rescale_is_one_rounded_fp32_multiply():
    rng = np.random.default_rng(2)
    x = F.bf16_value(F.bf16_from_f64(rng.standard_normal((4, 64)) * 30)).astype(np.float32)
    c = (1.0 + rng.integers(0, 8, 64) / 8.0) * np.ldexp(1.0, rng.integers(-3, 3, 64))
    c = c.astype(np.float32) * np.float32(1.0 + 2 ** -20)                # general fp32 values
    xt = rescale(x, c)
    for m in range(4):
        for k in range(64):
            exact = Fraction(float(x[m, k])) * Fraction(float(c[k]))
            v = xt[m, k]
            for nb in (np.nextafter(v, np.float32(-np.inf)), np.nextafter(v, np.float32(np.inf))):
                assert abs(Fraction(float(v)) - exact) <= abs(Fraction(float(nb)) - exact)


def _random_blocks(rng, R, K):
    x = rng.standard_normal((R, K)) * np.ldexp(1.0, rng.integers(-30, 30, (R, 1)))
    x[0, :8] = [0.25, 0.75, -1.25, 1.75, 2.5, -3.5, 5.0, 6.0]      # ties at unit 1 (amax 6 -> e=0)
    x[1, 16:20] = [2.0 ** -140, -2.0 ** -149, 0.0, -0.0]            # subnormals and zeros
    return x.astype(np.float32)


def _floor_log2_exact(a):
    f = Fraction(float(a))
    e = 0
    while Fraction(2) ** e > f:
        e -= 1
    while Fraction(2) ** (e + 1) <= f:
        e += 1
    return e


@pytest.mark.parametrize("fmt", ["mxfp4", "mxint4"])
def test_mx_brute_force(fmt):
    rng = np.random.default_rng(3)
    x = _random_blocks(rng, 6, 128)
    codes, scales, _ = quantize_rows(x, fmt)
    for m in range(x.shape[0]):
        for b in range(4):
            blk = x[m, 32 * b:32 * b + 32]
            amax = float(np.max(np.abs(blk)))
            e = -127 if amax == 0 else max(-127, min(127, _floor_log2_exact(amax) - 2))
            assert scales[m, b] == e + 127
            unit = Fraction(2) ** e
            for i, v in enumerate(blk):
                if fmt == "mxfp4":
                    want = _exact.e2m1_code(float(v), unit)
                else:
                    q = Fraction(float(v)) / unit
                    n = math.floor(q + Fraction(1, 2))
                    if q + Fraction(1, 2) == n and n % 2:       # exact tie -> even integer
                        n -= 1
                    want = max(-8, min(7, n)) & 15
                assert codes[m, 32 * b + i] == want, (m, b, i, v)


def test_nv_brute_force():
    rng = np.random.default_rng(4)
    x = _random_blocks(rng, 6, 64)
    x[2, :16] = x[2, :16] * np.float32(2.0 ** -60)       # a block whose scale rounds to 0
    codes, scales, t = quantize_rows(x, "nvfp4")
    tf = Fraction(float(t))
    assert t == np.float32(np.float32(np.max(np.abs(x))) / np.float32(2688))
    for m in range(x.shape[0]):
        for b in range(4):
            blk = x[m, 16 * b:16 * b + 16]
            amax = Fraction(float(np.max(np.abs(blk))))
            s = _exact.e4m3_code(amax / (6 * tf))
            assert scales[m, b] == s, (m, b)
            for i, v in enumerate(blk):
                if s == 0:
                    want = 8 if math.copysign(1.0, float(v)) < 0 else 0
                else:
                    want = _exact.e2m1_code(float(v), _exact.e4m3_exact(s) * tf)
                assert codes[m, 16 * b + i] == want, (m, b, i, v)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxint4", "nvfp4"])
def test_round_trip_of_representable_blocks(fmt):
    """A block built from codes and a scale, holding a largest-magnitude
    element, quantizes back to exactly those codes and that scale."""
    rng = np.random.default_rng(5)
    G = oracle.BLOCK[fmt]
    sbytes = list(range(90, 160, 3)) if fmt != "nvfp4" else list(range(8, 127, 4))
    t = np.float32(2.0 ** -4)
    rows, want_codes = [], []
    for s in sbytes:
        if fmt == "mxint4":
            c = rng.integers(-7, 8, G)
            c[rng.integers(G)] = 7
            vals = c * 2.0 ** (s - 127)
            want_codes.append(c & 15)
        else:
            c = rng.integers(0, 16, G)
            c[rng.integers(G)] = rng.choice([7, 15])
            unit = 2.0 ** (s - 127) if fmt == "mxfp4" else F.e4m3_value(s) * float(t)
            vals = F.e2m1_value(c) * unit
            want_codes.append(c)
        rows.append(vals)
    x = np.array(rows, np.float32)
    assert np.array_equal(x.astype(np.float64), np.array(rows))     # exactly representable
    codes, scales, _ = quantize_rows(x, fmt, t=t if fmt == "nvfp4" else None)
    assert scales[:, 0].tolist() == sbytes
    assert np.array_equal(codes, np.array(want_codes, np.uint8))


@pytest.mark.parametrize("fmt", ["mxfp4", "mxint4", "nvfp4"])
def test_scaling_by_power_of_two(fmt):
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((8, 128)) * 3).astype(np.float32)
    c0, s0, t0 = quantize_rows(x, fmt)
    for j in (-9, 1, 13):
        c1, s1, t1 = quantize_rows(x * np.float32(2.0 ** j), fmt)
        assert np.array_equal(c0, c1)
        if fmt == "nvfp4":
            assert np.array_equal(s0, s1) and t1 == t0 * np.float32(2.0 ** j)
        else:
            assert np.array_equal(s1.astype(int), s0.astype(int) + j)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxint4", "nvfp4"])
def test_negation(fmt):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((8, 128)) * 3).astype(np.float32)
    x[0, :4] = [7.5, 7.0, 0.0, 1.0]
    c0, s0, _ = quantize_rows(x, fmt)
    c1, s1, _ = quantize_rows(-x, fmt)
    assert np.array_equal(s0, s1)
    if fmt == "mxint4":
        v0, v1 = F.int4_value(c0), F.int4_value(c1)
        clipped = ((v0 == 7) & (v1 == -8)) | ((v0 == -8) & (v1 == 7))
        assert np.array_equal(v1[~clipped], -v0[~clipped])
        assert clipped.any()
    else:
        assert np.array_equal(c1, c0 ^ 8)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxint4", "nvfp4"])
def test_sign_preserving(fmt):
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((16, 256)) * 2).astype(np.float32)
    codes, scales, t = quantize_rows(x, fmt)
    deq = dequantize(pack_nibbles(codes), scales, fmt)
    nz = (x != 0) & (deq != 0)
    assert np.array_equal(np.sign(deq[nz]), np.sign(x[nz]))


def test_pack_layout():
    codes = np.arange(32, dtype=np.uint8).reshape(1, 32) & 15
    packed = pack_nibbles(codes)
    assert packed[0, :3].tolist() == [0x10, 0x32, 0x54]
    assert np.array_equal(unpack_nibbles(packed), codes)
