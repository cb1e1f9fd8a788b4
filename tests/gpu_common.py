"""Shared helpers of the GPU parity tests: device setup, oracle calls and the
comparison gates for the BF16 output.

Gates for Y (bf16) against the oracle's fp64 value y and its BF16 rounding Yr:
  G0  bit-exact Y == Yr where the fp32 accumulation is exact (all block
      scales of an operand equal, MX formats).
  G1  every element: |Y - y| <= 2^-8 |y| + (1 + 2^-8) E + 2^-133 with
      E = (K + 2) 2^-23 S + 2^-22 |y| and S = |r| t sum_k |a^_k w^_k| (the
      a-priori bound of an fp32 sum of K products in any order, the fp32
      epilogue multiplies, then one BF16 rounding).
  G2  each output row: ||Y - Yr||_2 / ||Yr||_2 <= 1e-3; an all-zero oracle
      row must be exactly zero.
BF16's own unit roundoff is 2^-8 (3.9e-3), so no elementwise 1e-3 bound
against the unrounded value is attainable; G2 is the 1e-3 reading that is.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
import w4a4_block_scaled_amd as w4

REL_TOL = 1e-3


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(w4.library_path()):
        pytest.fail("libw4a4.so is not built; GPU tests need the HIP library (no fallback)")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a, dev):
    if isinstance(a, torch.Tensor):
        return a.contiguous().to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def gpu_quantize(x_bf16, c, fmt, dev):
    codes, scales, t = w4.quantize_act(to_dev(x_bf16, dev), None if c is None else to_dev(c, dev), fmt)
    torch.cuda.synchronize()
    return codes, scales, t


def check_linear(Y_bits, y, S, K, label=""):
    """Apply gates G1 and G2; returns (max elementwise rel err vs y, max row rel L2)."""
    yhat = F.bf16_value(Y_bits)
    assert np.isfinite(yhat).all(), f"{label}: non-finite outputs"
    ay = np.abs(y)
    E = (K + 2) * 2.0 ** -23 * S + 2.0 ** -22 * ay
    bound = 2.0 ** -8 * ay + (1 + 2.0 ** -8) * E + 2.0 ** -133
    err = np.abs(yhat - y)
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: G1 violated at {tuple(i)}: gpu={yhat[tuple(i)]!r} "
                             f"oracle={y[tuple(i)]!r} bound={bound[tuple(i)]!r} ({bad.sum()} elements)")
    Yr = F.bf16_value(F.bf16_from_f64(y))
    num = np.linalg.norm(yhat - Yr, axis=1)
    den = np.linalg.norm(Yr, axis=1)
    zero = den == 0
    assert np.all(num[zero] == 0), f"{label}: nonzero output where the oracle row is zero"
    rel = np.where(zero, 0.0, num / np.where(zero, 1.0, den))
    assert rel.max() <= REL_TOL, f"{label}: G2 row rel-L2 {rel.max():.3e} > {REL_TOL}"
    nz = ay > 0
    elem = float(np.max(err[nz] / ay[nz])) if nz.any() else 0.0
    return elem, float(rel.max())
