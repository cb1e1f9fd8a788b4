"""Block quantization of rows, activation and weight side (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed (DualQuant):

* Section 4.2, eq. (3) "column scales as activation rescalings": the tensor
  that gets quantized at inference is X~ = X Diag(beta)^-1.  Writing the
  stored inverse column scale as c = beta^-1 (the admissible set holds the
  inverse scales, Section 4.2), X~[m,k] = X[m,k] * c[k]; here one fp32
  multiply of the BF16 input, rounded to nearest even.
* Section 4.4: Q(X~) is the format-native row-wise quantization: rows are
  tokens, each row is cut along K into blocks of G contiguous elements
  (Section 3, block-wise quantization), every block gets its own scale.
* Section 3: Q(W) = Delta * proj_G(W / Delta) with proj_G rounding to the
  nearest grid point and clipping.  The scale of a block:
    - MX formats (E8M0): the OCP microscaling shared-exponent rule the
      section cites, e = floor(log2 amax) - emax_elem with emax_elem = 2 for
      E2M1 (largest element 6 = 1.5 * 2^2) and the same offset for INT4
      codes -8..7, clamped to the E8M0 range [-127, 127].  An all-zero block
      gets byte 0.
    - NVFP4 (UE4M3): s = RNE_E4M3(amax / (6 t)), saturating at 448, where the
      FP32 tensor scale t = fp32(max|X~|) / 2688 (one fp32 division;
      2688 = 6 * 448 so the largest block lands on the largest scale); t = 1
      when the tensor is all zero (or when that division underflows to 0).
      This tensor scale is not defined on the pages; it is this library's
      reading of the NVFP4 per-tensor scale.
* Elements: MXFP4 code = RNE_E2M1(x~ * 2^-e); MXINT4 code =
  clip(RNE(x~ * 2^-e), -8, 7); NVFP4 code = RNE_E2M1(x~ / (s t)), all
  decided exactly.  NVFP4 blocks whose scale rounds to 0 keep only the sign.
* INT4 with G = 64 and BF16 block scales (the paper's packed deployment
  format, Section 4.2 "admissible sets" with BF16 for INT4; Section 3's
  symmetric scale Delta = max|x| / q_max with q_max = 7 for INT4):
  Delta = BF16(amax / 7), rounded once to nearest even from the exact
  quotient; code = clip(RNE(x~ / Delta), -8, 7) decided exactly (ties to
  the even integer); an all-zero block (or one whose Delta rounds to 0)
  gets Delta = 0 and zero codes.
* INT8 with G = 128 and BF16 block scales (Appendix G.2, Table 9's 8-bit
  integer W+A variant, G = 128 on both operands): Section 3's symmetric scale
  with q_max = 127, Delta = BF16(amax / 127) rounded once to nearest even
  from the exact quotient (BF16 scales read as for INT4 G=64: the pages give
  no other scale format for the integer grid); code = clip(RNE(x~ / Delta),
  -128, 127), the whole two's-complement grid (only a subnormal Delta, which
  rounds far from amax / 127, can take a code past +-127); zero blocks and
  non-finite blocks as for INT4 G=64.  Codes are stored one byte per
  element, [rows, K].
* 8-bit MX formats (Appendix G.2, Table 9: MXFP8 and MXINT8 with G = 32 and
  E8M0 scales), with the same OCP shared-exponent rule: MXFP8 elements are
  E4M3 (emax_elem = 8, 448 = 1.75 * 2^8), code = RNE_E4M3(x~ * 2^-e)
  saturating at +-448, sign kept for -0 (0x80); MXINT8 elements are
  two's-complement bytes with value code * 2^e, emax_elem = 6 (127 < 2^7),
  code = clip(RNE(x~ * 2^-e), -128, 127) (the OCP fixed-point convention
  with 6 fraction bits gives the same values with the scale byte 6 higher).
  Codes are stored one byte per element, [rows, K].
* MX and INT4 G=64 / INT8 G=128 blocks holding a non-finite value get scale
  byte 0xFF (BF16 0x7FC0) and zero codes (inputs are expected finite; this
  only fixes what happens otherwise).

Canonical storage: codes [rows, K/2] bytes, element 2j in the low nibble of
byte j and 2j+1 in the high nibble; scales [rows, K/G] bytes, row-major
(uint16 BF16 bit patterns for INT4 G=64 and INT8 G=128).
"""
from __future__ import annotations

import numpy as np

from . import formats as F

BLOCK = {"mxfp4": 32, "nvfp4": 16, "mxint4": 32, "int4g64": 64, "mxfp8": 32, "mxint8": 32,
         "int8g128": 128}
MX_FORMATS = ("mxfp4", "mxint4", "mxfp8", "mxint8")
CODE_BITS = {"mxfp4": 4, "nvfp4": 4, "mxint4": 4, "int4g64": 4, "mxfp8": 8, "mxint8": 8,
             "int8g128": 8}
BF16_SCALED = ("int4g64", "int8g128")   # integer grids with BF16 block scales
INT4_QMAX = 7                      # symmetric INT4 grid maximum
INT8_QMAX = 127                    # symmetric INT8 grid maximum
# floor(log2) of the largest element magnitude of each MX element grid:
# E2M1 6 = 1.5 * 2^2; int4 7 < 2^3; E4M3 448 = 1.75 * 2^8; int8 127 < 2^7
EMAX_ELEM = {"mxfp4": 2, "mxint4": 2, "mxfp8": 8, "mxint8": 6}
NV_TENSOR_DIVISOR = np.float32(6.0 * 448.0)   # 2688
ROW_CHUNK = 256


def rescale(x, c):
    """X~ = fp32(X) * c[k], one correctly rounded fp32 multiply (eq. 3)."""
    x = np.asarray(x, np.float32)
    c = np.asarray(c, np.float32)
    return (x * c[None, :]).astype(np.float32)


def nv_tensor_scale(xt):
    """FP32 per-tensor scale t = fp32(max|X~|) / 2688 for NVFP4."""
    amax = np.float32(np.max(np.abs(np.asarray(xt, np.float32)))) if np.size(xt) else np.float32(0)
    t = np.float32(amax / NV_TENSOR_DIVISOR)
    if amax == 0 or t == 0:
        t = np.float32(1.0)
    return t


def _mx_scale_exponent(amax, emax_elem=2):
    """Shared exponent e = clamp(floor(log2 amax) - emax_elem, -127, 127); 0 blocks -> -127."""
    _, E = np.frexp(amax)                       # amax = f * 2^E, f in [0.5, 1)
    e = np.clip(E - 1 - emax_elem, -127, 127)
    return np.where(amax == 0, -127, e).astype(np.int64)


def _quantize_chunk(xt, fmt, t):
    R, K = xt.shape
    G = BLOCK[fmt]
    blocks = xt.astype(np.float64).reshape(R, K // G, G)
    amax = np.abs(blocks).max(axis=-1)
    if fmt in MX_FORMATS:
        nonfinite = ~np.isfinite(blocks).all(axis=-1)
        amax = np.where(nonfinite, 0.0, amax)
        e = _mx_scale_exponent(amax, EMAX_ELEM[fmt])
        scales = (e + 127).astype(np.uint8)
        finite = np.where(np.isfinite(blocks), blocks, 0.0)
        if fmt == "mxfp4":
            codes = F.e2m1_encode(blocks, np.ldexp(1.0, e)[..., None])
        elif fmt == "mxfp8":
            codes = F.e4m3_encode(finite, np.ldexp(1.0, e)[..., None])
        elif fmt == "mxint8":
            codes = F.int8_encode(np.clip(np.rint(np.ldexp(finite, -e[..., None])), -128, 127))
        else:
            v = np.ldexp(finite, -e[..., None])
            codes = F.int4_encode(np.clip(np.rint(v), -8, 7))
        scales = np.where(nonfinite, np.uint8(255), scales)
        codes = np.where(nonfinite[..., None], np.uint8(0), codes)
    elif fmt in BF16_SCALED:
        qmax = INT4_QMAX if fmt == "int4g64" else INT8_QMAX
        nonfinite = ~np.isfinite(blocks).all(axis=-1)
        amax = np.where(nonfinite, 0.0, amax)
        # amax / q_max in fp64 then one rounding to BF16: the fp64 quotient can
        # only land on a BF16 midpoint when the exact quotient is that
        # midpoint, so this is the single correct rounding of amax / q_max
        bits = F.bf16_from_f64(amax / qmax)
        delta = F.bf16_value(bits)
        live = delta > 0
        # x~ (24 bits) / Delta (8 bits) in fp64: a quotient that is not a
        # half-integer differs from one by far more than the fp64 rounding,
        # so rint of the fp64 quotient is the exact nearest-even decision
        with np.errstate(invalid="ignore", over="ignore"):
            v = np.where(live[..., None] & np.isfinite(blocks),
                         blocks / np.where(live, delta, 1.0)[..., None], 0.0)
        if fmt == "int4g64":
            codes = F.int4_encode(np.clip(np.rint(v), -8, 7))
        else:
            codes = F.int8_encode(np.clip(np.rint(v), -128, 127))
        scales = np.where(nonfinite, np.uint16(0x7FC0), np.where(live, bits, np.uint16(0)))
        codes = np.where(nonfinite[..., None], np.uint8(0), codes)
        return codes.reshape(R, K).astype(np.uint8), scales.astype(np.uint16)
    else:
        den = 6.0 * np.float64(t)                  # exact: 2 + 24 significant bits
        scales = F.e4m3_encode_ratio(amax, den)
        unit = F.e4m3_value(scales) * np.float64(t)   # exact: 4 + 24 bits
        zero_scale = scales == 0
        safe_unit = np.where(zero_scale, 1.0, unit)
        codes = F.e2m1_encode(blocks, safe_unit[..., None])
        sign_only = (np.signbit(blocks).astype(np.uint8) << 3)
        codes = np.where(zero_scale[..., None], sign_only, codes)
    return codes.reshape(R, K).astype(np.uint8), scales.astype(np.uint8)


def quantize_rows(xt, fmt, t=None):
    """Quantize the rows of X~ (fp32 [R, K]) -> (codes [R,K], scales [R,K/G], t).

    codes hold one element each: a nibble for the 4-bit formats, a byte for
    MXFP8 / MXINT8.

    t is the NVFP4 tensor scale (computed from X~ when not given); None for
    MX formats.
    """
    xt = np.asarray(xt, np.float32)
    R, K = xt.shape
    G = BLOCK[fmt]
    if K % G:
        raise ValueError(f"K={K} is not a multiple of the block size {G}")
    if fmt == "nvfp4" and t is None:
        t = nv_tensor_scale(xt)
    codes = np.empty((R, K), np.uint8)
    scales = np.empty((R, K // G), np.uint16 if fmt in BF16_SCALED else np.uint8)
    for r0 in range(0, R, ROW_CHUNK):
        codes[r0:r0 + ROW_CHUNK], scales[r0:r0 + ROW_CHUNK] = \
            _quantize_chunk(xt[r0:r0 + ROW_CHUNK], fmt, t)
    return codes, scales, (np.float32(t) if fmt == "nvfp4" else None)


def pack_codes(codes, fmt):
    """Canonical storage of element codes: nibble pairs for 4-bit formats
    (pack_nibbles), the bytes themselves for the 8-bit formats."""
    return pack_nibbles(codes) if CODE_BITS[fmt] == 4 else np.asarray(codes, np.uint8).copy()


def unpack_codes(packed, fmt):
    return unpack_nibbles(packed) if CODE_BITS[fmt] == 4 else np.asarray(packed, np.uint8).copy()


def pack_nibbles(codes):
    """[R, K] nibbles -> [R, K/2] bytes, even element in the low nibble."""
    codes = np.asarray(codes, np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    packed = np.asarray(packed, np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), np.uint8)
    out[:, 0::2] = packed & 15
    out[:, 1::2] = packed >> 4
    return out


def quantize_act(x, c, fmt):
    """Activation side: rescale by c then quantize rows.

    x : fp32 values of the BF16 activations [M, K]; c : fp32 [K].
    Returns (packed codes [M, K/2] (8-bit formats: [M, K]), scales [M, K/G],
    t or None).
    """
    codes, scales, t = quantize_rows(rescale(x, c), fmt)
    return pack_codes(codes, fmt), scales, t


def quantize_weight(w, fmt):
    """Weight side: quantize rows of the already divided weights W / (r c^T).

    w : fp32 values of the BF16 prescaled weights [N, K].
    Returns (packed codes [N, K/2] (8-bit formats: [N, K]), scales [N, K/G],
    t_w (1.0 for MX)).
    """
    codes, scales, t = quantize_rows(np.asarray(w, np.float32), fmt)
    return pack_codes(codes, fmt), scales, (np.float32(1.0) if t is None else t)


def dequantize(packed, scales, fmt):
    """Values code * block_scale in fp64 (exact); the NVFP4 tensor scale is not applied."""
    codes = unpack_codes(packed, fmt)
    R, K = codes.shape
    G = BLOCK[fmt]
    if fmt in ("mxint4", "int4g64"):
        elem = F.int4_value(codes)
    elif fmt == "mxfp8":
        elem = F.e4m3_value(codes)
    elif fmt in ("mxint8", "int8g128"):
        elem = F.int8_value(codes)
    else:
        elem = F.e2m1_value(codes)
    if fmt in BF16_SCALED:
        svals = F.bf16_value(scales)
    elif fmt in MX_FORMATS:
        svals = F.e8m0_value(scales)
    else:
        svals = F.e4m3_value(scales)
    return (elem.reshape(R, K // G, G) * svals[..., None]).reshape(R, K)
