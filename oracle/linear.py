"""The fake-quantized W4A4 linear (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

DualQuant, Section 4.4: the layer computes Q(X~) Q^T Diag(alpha)^-1.  With
the stored inverse row scale r = alpha^-1 this is

    Y[m, n] = r[n] * sum_k  A^[m, k] * W^[n, k]

where A^ and W^ are the dequantized operands (code times block scale, times
the tensor scale for NVFP4).  The paper checks its packed kernels against
exactly this kind of fake quantization (Appendix I, "Accuracy").  Here the
products are summed in fp64 (a numpy matmul serves as the sum) and the result
is rounded once from fp64 to BF16.
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from .quant import dequantize, quantize_act, quantize_weight


def linear_f64(a_codes, a_scales, t_a, w_codes, w_scales, t_w, r, fmt):
    """fp64 result y[m, n] before the BF16 rounding."""
    A = dequantize(a_codes, a_scales, fmt)          # [M, K]
    W = dequantize(w_codes, w_scales, fmt)          # [N, K]
    P = A @ W.T
    if fmt == "nvfp4":
        P = P * (np.float64(t_a) * np.float64(t_w))
    return P * np.asarray(r, np.float64)[None, :]


def linear(a_codes, a_scales, t_a, w_codes, w_scales, t_w, r, fmt):
    """BF16 output bits [M, N] (uint16) and the fp64 value they round."""
    y = linear_f64(a_codes, a_scales, t_a, w_codes, w_scales, t_w, r, fmt)
    return F.bf16_from_f64(y), y


def linear_abs_sum(a_codes, a_scales, t_a, w_codes, w_scales, t_w, r, fmt):
    """|r[n]| * sum_k |A^[m,k] W^[n,k]| in fp64: the scale of the error bound."""
    A = np.abs(dequantize(a_codes, a_scales, fmt))
    W = np.abs(dequantize(w_codes, w_scales, fmt))
    P = A @ W.T
    if fmt == "nvfp4":
        P = P * (np.float64(t_a) * np.float64(t_w))
    return P * np.abs(np.asarray(r, np.float64))[None, :]


def layer(x, c, w_codes, w_scales, t_w, r, fmt):
    """Whole hot path for one linear: rescale+quantize X, then the linear."""
    a_codes, a_scales, t_a = quantize_act(x, c, fmt)
    bits, y = linear(a_codes, a_scales, t_a, w_codes, w_scales, t_w, r, fmt)
    return a_codes, a_scales, t_a, bits, y


def layer_prescaled(x, c, w_prescaled, r, fmt):
    """As layer(), with the weights given as W / (r c^T) still to be quantized."""
    w_codes, w_scales, t_w = quantize_weight(w_prescaled, fmt)
    return (w_codes, w_scales, t_w) + layer(x, c, w_codes, w_scales, t_w, r, fmt)
