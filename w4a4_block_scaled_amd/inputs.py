"""Seeded synthetic workloads for the packed W4A4 linear.

This module only draws random numbers and lays them out; it contains none
of the quantization arithmetic (no rescale, no block amax, no scale or
element encoding, no GEMM).  Both the GPU path and the CPU oracle consume
exactly what it returns, so every parity test and benchmark sees the same
bits on both sides.

Workloads (DualQuant, "Experiments" and Appendix I: Llama-3.1-8B and
Qwen-7B-class linears; formats MXFP4 / NVFP4 / MXINT4 from Section 3):

* ``single``  : one MXFP4 linear, M=16, N=K=256.  Weight codes are drawn
  directly (uniform over all 16 nibbles) with E8M0 block exponents uniform
  in {-6..1}; activations N(0,1) with 2 outlier channels x50; r and c drawn
  from lognormal(0, 0.5) as continuous fp32 values.
* ``llama_decode`` / ``llama_prefill`` : MXFP4, M in {1,4,16} / 2048, the
  four Llama-3.1-8B linears (QKV 4096->6144, O 4096->4096, gate+up
  4096->28672, down 14336->4096).  Raw weights N(0, 0.02) are divided by
  r and c (the dual-scale parameterization, Section 4.2 eq. 2) and handed
  over as BF16; the method's own quantizer turns them into codes.
  Activations N(0,1) with round(0.01 K) outlier channels x30.
* ``llama_nvfp4`` : NVFP4, M=4096, same shapes; activations i.i.d.
  Student-t with 3 degrees of freedom.
* ``llama_mxfp8`` / ``llama_mxint8`` : the 8-bit MX variants (Appendix G.2),
  M in {2048, 1}, Llama shapes and laws as ``llama_prefill``.
* ``llama_int8g128`` : INT8 with G = 128 and BF16 block scales (Appendix
  G.2's 8-bit integer variant), M in {2048, 1}, as ``llama_mxfp8``; r and c
  lognormal(0, 0.5) rounded to BF16.
* ``qwen_mxint4`` : MXINT4, M in {1,512,4096}, Qwen-7B-class shapes (QKV
  3584->4608, O 3584->3584, gate+up 3584->37888, down 18944->3584).
  Weight codes drawn directly (uniform int4) with E8M0 exponents uniform in
  {-7..1}; activations N(0,1) with round(2K/256) outlier channels x50.

Row and column scales r, c of the other workloads follow a lognormal(0, 0.5)
law sampled on the admissible set of the format (Section 4.2: inverse scales live in E8M0 for
MX formats, UE4M3 for NVFP4): for E8M0 the power-of-two exponent is a
normal draw with standard deviation 0.5/ln 2 rounded to an integer; for
UE4M3 the binade is the floor of that draw and the 3-bit mantissa is
uniform.  Drawing directly on the set keeps the projection (part of the
offline solver, not of the inference path) out of this module.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

FORMATS = ("mxfp4", "nvfp4", "mxint4", "int4g64", "mxfp8", "mxint8", "int8g128")
BLOCK = {"mxfp4": 32, "nvfp4": 16, "mxint4": 32, "int4g64": 64, "mxfp8": 32, "mxint8": 32,
         "int8g128": 128}
EIGHT_BIT = ("mxfp8", "mxint8", "int8g128")

LLAMA_LINEARS = (("qkv", 6144, 4096), ("o", 4096, 4096),
                 ("gate_up", 28672, 4096), ("down", 4096, 14336))
QWEN_LINEARS = (("qkv", 4608, 3584), ("o", 3584, 3584),
                ("gate_up", 37888, 3584), ("down", 3584, 18944))

WORKLOADS = {
    # name: (seed, fmt, default M list, linears)
    "single": (1, "mxfp4", (16,), (("single", 256, 256),)),
    "llama_decode": (2, "mxfp4", (1, 4, 16), LLAMA_LINEARS),
    "llama_prefill": (3, "mxfp4", (2048,), LLAMA_LINEARS),
    "llama_nvfp4": (4, "nvfp4", (4096,), LLAMA_LINEARS),
    "qwen_mxint4": (5, "mxint4", (1, 512, 4096), QWEN_LINEARS),
    # INT4 G=64 with BF16 scales: Llama shapes, prefill and decode
    "llama_int4g64": (6, "int4g64", (2048, 1), LLAMA_LINEARS),
    # the 8-bit MX variants (Appendix G.2, Table 9): Llama shapes, prefill and decode
    "llama_mxfp8": (7, "mxfp8", (2048, 1), LLAMA_LINEARS),
    "llama_mxint8": (8, "mxint8", (2048, 1), LLAMA_LINEARS),
    # INT8 with G = 128 and BF16 scales (Table 9's 8-bit integer variant)
    "llama_int8g128": (9, "int8g128", (2048, 1), LLAMA_LINEARS),
}


@dataclasses.dataclass
class LinearCase:
    """One linear layer's synthetic inputs.

    x           : torch.bfloat16 [M, K] (CPU)
    c           : float32 [K]  column scales (multiplied into x)
    r           : float32 [N]  row scales (multiplied into the output)
    w_prescaled : torch.bfloat16 [N, K] weights already divided by r and c,
                  to be quantized by the method's quantizer (or None)
    w_codes     : uint8 [N, K/2] canonical packed codes ([N, K] for 8-bit
                  formats) (or None)
    w_scales    : uint8 [N, K/G] block scale bytes (uint16 BF16 patterns for
                  int4g64 and int8g128) (or None)
    t_w         : float tensor scale of the weights when codes are drawn
    """
    workload: str
    name: str
    fmt: str
    M: int
    N: int
    K: int
    x: torch.Tensor
    c: np.ndarray
    r: np.ndarray
    w_prescaled: Optional[torch.Tensor] = None
    w_codes: Optional[np.ndarray] = None
    w_scales: Optional[np.ndarray] = None
    t_w: float = 1.0

    @property
    def G(self) -> int:
        return BLOCK[self.fmt]


def _rngs(seed: int, n: int) -> List[np.random.Generator]:
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """float32 array -> torch.bfloat16 (round to nearest even, torch's cast)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def admissible_scales(rng: np.random.Generator, n: int, family: str) -> np.ndarray:
    """Draw n positive scales from a lognormal(0, 0.5) law on an admissible set."""
    z = rng.standard_normal(n) * (0.5 / math.log(2.0))
    if family == "e8m0":
        return np.ldexp(1.0, np.rint(z).astype(np.int64)).astype(np.float32)
    if family == "ue4m3":
        e = np.floor(z).astype(np.int64)
        m = rng.integers(0, 8, n)
        return np.ldexp(1.0 + m / 8.0, e).astype(np.float32)
    if family == "bf16":
        return to_bf16(np.exp(z * math.log(2.0)).astype(np.float32)).float().numpy()
    raise ValueError(family)


def lognormal_scales(rng: np.random.Generator, n: int) -> np.ndarray:
    """n draws of exp(N(0, 0.5^2)) as fp32 (not restricted to an admissible set)."""
    return np.exp(rng.standard_normal(n) * 0.5).astype(np.float32)


def scale_family(fmt: str) -> str:
    return {"nvfp4": "ue4m3", "int4g64": "bf16", "int8g128": "bf16"}.get(fmt, "e8m0")


def random_codes_bf16(rng: np.random.Generator, N: int, K: int, exp_lo: int, exp_hi: int):
    """Canonical packed codes uniform over all 16 nibbles and BF16 block scales
    2^e (1 + m/128), e in U{lo..hi}, m in U{0..127} (uint16 bit patterns, G = 64)."""
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    e = rng.integers(exp_lo, exp_hi + 1, size=(N, K // 64))
    m = rng.integers(0, 128, size=(N, K // 64))
    return codes, (((127 + e) << 7) | m).astype(np.uint16)


def outlier_activations(rng: np.random.Generator, M: int, K: int, n_out: int,
                        factor: float) -> torch.Tensor:
    x = rng.standard_normal((M, K), dtype=np.float32)
    if n_out:
        cols = rng.choice(K, size=n_out, replace=False)
        x[:, cols] *= np.float32(factor)
    return to_bf16(x)


def student_t_activations(rng: np.random.Generator, M: int, K: int) -> torch.Tensor:
    return to_bf16(rng.standard_t(3.0, size=(M, K)).astype(np.float32))


def prescaled_weights(rng: np.random.Generator, N: int, K: int, r: np.ndarray,
                      c: np.ndarray) -> torch.Tensor:
    """N(0, 0.02) weights divided by r[n] c[k] (fp64, rounded to fp32, then BF16)."""
    w = rng.standard_normal((N, K), dtype=np.float32).astype(np.float64) * 0.02
    w /= r.astype(np.float64)[:, None]
    w /= c.astype(np.float64)[None, :]
    return to_bf16(w.astype(np.float32))


def random_codes(rng: np.random.Generator, N: int, K: int, G: int,
                 exp_lo: int, exp_hi: int, fmt: str = "mxfp4"):
    """Canonical codes and E8M0 bytes 127+U{lo..hi}: packed nibbles uniform over
    all 16 values, or for the 8-bit formats one byte per element, uniform over
    all 256 bytes except the E4M3 NaN codes 0x7F / 0xFF (MXFP8).  INT8 G=128
    takes BF16 block scales 2^e (1 + m/128), e in U{lo..hi}, m in U{0..127}."""
    if fmt == "int8g128":
        codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
        e = rng.integers(exp_lo, exp_hi + 1, size=(N, K // G))
        m = rng.integers(0, 128, size=(N, K // G))
        return codes, (((127 + e) << 7) | m).astype(np.uint16)
    if fmt in EIGHT_BIT:
        codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
        if fmt == "mxfp8":
            codes = np.where((codes & 0x7F) == 0x7F, codes - 1, codes).astype(np.uint8)
    else:
        codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = (127 + rng.integers(exp_lo, exp_hi + 1, size=(N, K // G))).astype(np.uint8)
    return codes, scales


def make_case(workload: str, name: str, fmt: str, M: int, N: int, K: int,
              seed: int, build_weights: bool = True) -> LinearCase:
    """Build one linear of a workload; the seed fixes every tensor."""
    rx, rc, rr, rw = _rngs(seed, 4)
    G = BLOCK[fmt]
    if workload == "single":
        # the single-linear configuration draws r and c from the lognormal law
        # itself (continuous fp32 values), so the activation rescale is a
        # rounded fp32 product
        c = lognormal_scales(rc, K)
        r = lognormal_scales(rr, N)
    else:
        family = scale_family(fmt)
        c = admissible_scales(rc, K, family)
        r = admissible_scales(rr, N, family)
    if workload == "llama_nvfp4":
        x = student_t_activations(rx, M, K)
    elif workload in ("llama_decode", "llama_prefill", "llama_int4g64", "llama_mxfp8", "llama_mxint8",
                      "llama_int8g128"):
        x = outlier_activations(rx, M, K, int(round(0.01 * K)), 30.0)
    else:  # single, qwen_mxint4 and ad-hoc cases: the single-linear distributions
        x = outlier_activations(rx, M, K, int(round(2 * K / 256)), 50.0)
    case = LinearCase(workload, name, fmt, M, N, K, x, c, r)
    if not build_weights:
        return case
    if workload == "llama_int4g64":
        case.w_codes, case.w_scales = random_codes_bf16(rw, N, K, -9, -6)
    elif workload in ("single", "qwen_mxint4"):
        lo = -6 if fmt == "mxfp4" else -7
        case.w_codes, case.w_scales = random_codes(rw, N, K, G, lo, 1)
    else:
        case.w_prescaled = prescaled_weights(rw, N, K, r, c)
    return case


def workload_cases(workload: str, M: Optional[int] = None,
                   linears: Optional[Sequence[str]] = None,
                   build_weights: bool = True) -> List[LinearCase]:
    """All linears of a named workload at token count M (default: first listed M)."""
    seed, fmt, Ms, lins = WORKLOADS[workload]
    M = Ms[0] if M is None else M
    out = []
    for i, (name, N, K) in enumerate(lins):
        if linears is not None and name not in linears:
            continue
        out.append(make_case(workload, name, fmt, M, N, K, seed * 1000 + i * 17 + M,
                             build_weights))
    return out


def adhoc_case(fmt: str, M: int, N: int, K: int, seed: int,
               weights: str = "prescaled") -> LinearCase:
    """A case of any shape with the single-linear activation law.

    weights = "prescaled" (N(0,0.02)/(r c), quantized by the method),
    "codes" (random codes with block exponents in {-6..1}; MX formats and
    INT8 G=128) or "none".
    """
    rx, rc, rr, rw = _rngs(seed, 4)
    family = scale_family(fmt)
    c = admissible_scales(rc, K, family)
    r = admissible_scales(rr, N, family)
    x = outlier_activations(rx, M, K, int(round(2 * K / 256)), 50.0)
    case = LinearCase("adhoc", f"adhoc_{M}x{N}x{K}", fmt, M, N, K, x, c, r)
    if weights == "none":
        return case
    if weights == "codes":
        case.w_codes, case.w_scales = random_codes(rw, N, K, BLOCK[fmt], -6, 1, fmt)
    else:
        case.w_prescaled = prescaled_weights(rw, N, K, r, c)
    return case
