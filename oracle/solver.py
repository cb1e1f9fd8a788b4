"""DualQuant's offline dual-scale solver (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is minimized (DualQuant Section 4.3, eq. 4): the weight-reconstruction
error

    E(alpha, beta) = || W - Diag(alpha)^-1 Q(Diag(alpha) W Diag(beta)) Diag(beta)^-1 ||_F^2

over a row scale alpha (one per output row) and a column scale beta (one per
input column) whose inverses r = alpha^-1 and c = beta^-1 lie in the
format's admissible set F (Section 4.2: E8M0 for the MX formats, UE4M3 for
NVFP4).  Q is the format's row-wise block quantizer (Section 3;
`quant.quantize_rows`; for NVFP4 with the fp32 tensor scale of the tensor it
quantizes), and Q^ below is its value (code x block scale, x t for NVFP4).

How (block coordinate descent with variable splitting, Section 4.3 and
Appendices A-B, Algorithm 1 of the paper): with the quantized matrix Q^ held
fixed, E is a sum of independent 1-D quadratics in the inverse scales of one
axis, u = r_i along rows or v = c_j along columns,

    || W_slice - u * D_slice ||^2,   D = Q^ / (the other axis' scale),

whose minimizer is <W_slice, D_slice> / ||D_slice||^2 (Appendix B); the
nearest admissible value is then the constrained minimizer (Appendix C,
Remark 1).  One generic half-step, `half_step`, does this for one axis: it
re-quantizes at the current scales (the inner copies are synchronized with
the outer ones, Appendix A.1), then sets that axis' scales.  An iteration is
the row half-step followed by the column half-step; T = 15 iterations by
default (Section 5), stopping early when an iteration leaves (alpha, beta)
unchanged, since every later iteration would then repeat it exactly.

Readings where the pages leave a step open:
  * Initialization (Section 5, "Hyperparameter selection": the row absmax and
    the column l1 norm).  Read with the inverse-scale convention of Section
    4.2: alpha_0^-1 = max_j |W_ij| and beta_0^-1 = sum_i |W_ij|, so beta_0
    equalizes the columns.  This is the reading under which beta reproduces
    Table 5 (beta correlates with SmoothQuant's weight-only scale
    1 / max_i |W_ij|, Pearson 0.83-0.97 there; pinned by outcome in the
    tests); taking the magnitudes as the multipliers themselves gives a
    negative correlation, and starting from alpha = beta = 1 none.  alpha_0 =
    fp32(1 / absmax), beta_0 = fp32(1 / l1) from fp64 quotients; an all-zero
    row or column starts at 1.  These starting scales are not admissible;
    the first half-steps project them.
  * The rescaled weight is W~_ij = fp32(fp32(alpha_i * W_ij) * beta_j), with
    alpha = fp32(1 / r) and beta = fp32(1 / c) (fp64 quotients rounded to
    fp32; exact for E8M0) and fp32 W.  For NVFP4, Q^ includes the tensor
    scale t of W~ (code x block scale x t, exact in fp64), and the returned
    codes come with the t of the final W~ (t_w; 1 for the MX formats).
  * Q^ and D are fp64 values (Q^ exact, D one fp64 division each); the inner
    products and squared norms are exact sums of the fp64 products
    (math.fsum), rounded once.
  * The projection is to the nearest admissible value in linear distance
    (Remark 1: the subproblem is a convex quadratic in the inverse scale).
    E8M0: the powers of two 2^e, e in [-127, 127]; an exact tie 1.5 * 2^e
    goes to 2^(e+1); a non-positive minimizer goes to 2^-127.  UE4M3: the
    126 positive finite E4M3 values (zero would zero the row); ties go to
    the even code, as in E4M3 rounding; above 448 saturates; a minimizer
    below 2^-9 (or non-positive) goes to 2^-9.
  * A row (column) whose Q^ is all zero has no minimizer; its scale is set to
    1 (the pages' convention for rows, applied to columns alike).

What follows from these readings (recorded, and pinned where the pages fix
an outcome): for the MX formats a power-of-two row scale is absorbed by the
E8M0 block scales (Q(2^k x) = 2^k Q(x)), so row half-steps change the row
scales but not the reconstruction (Table 4 shows the alpha-only variant equal
to RTN on MXFP4 for the same reason); the column update fits the scale to
values quantized at the current scale, so it moves only where quantization
bias pushes the least-squares coefficient past a projection midpoint, and
(alpha, beta) reach a fixed point within a few iterations.
"""
from __future__ import annotations

import math

import numpy as np

from .quant import quantize_rows, pack_nibbles, dequantize

E8M0_MIN = 2.0 ** -127
E8M0_MAX = 2.0 ** 127


def project_e8m0(u):
    """Nearest power of two 2^e (e in [-127, 127]) to u in linear distance."""
    u = np.asarray(u, np.float64)
    pos = u > 0
    _, e = np.frexp(np.where(pos, u, 1.0))          # 2^(e-1) <= u < 2^e
    lo = np.ldexp(1.0, (e - 1).astype(np.int64))
    with np.errstate(over="ignore"):
        near = np.where(u >= 1.5 * lo, 2.0 * lo, lo)
    return np.where(pos, np.clip(near, E8M0_MIN, E8M0_MAX), E8M0_MIN)


E4M3_POS = np.array([np.ldexp(float(m), -9) if e == 0 else np.ldexp(float(8 + m), e - 10)
                     for e in range(16) for m in range(8)])[1:127]   # codes 1 .. 126


def project_ue4m3(u):
    """Nearest positive finite E4M3 value to u in linear distance, ties to the even code."""
    u = np.asarray(u, np.float64)
    i = np.clip(np.searchsorted(E4M3_POS, u), 1, len(E4M3_POS) - 1)  # E4M3_POS[i-1] < u <= E4M3_POS[i]
    lo, hi = E4M3_POS[i - 1], E4M3_POS[i]
    mid = 0.5 * (lo + hi)                                            # exact in fp64
    code_lo = i                                                      # E4M3 code of lo is i (codes start at 1)
    pick_hi = (u > mid) | ((u == mid) & (code_lo % 2 == 1))
    out = np.where(pick_hi, hi, lo)
    out = np.where(u >= E4M3_POS[-1], E4M3_POS[-1], out)
    return np.where(u > E4M3_POS[0], out, E4M3_POS[0])


def project(u, fmt):
    return project_ue4m3(u) if fmt == "nvfp4" else project_e8m0(u)


def exact_sums(P, axis):
    """Correctly rounded sums of the fp64 array P along `axis` (math.fsum)."""
    P = np.asarray(P, np.float64)
    P = P if axis == 1 else P.T
    return np.array([math.fsum(row) for row in P], np.float64)


def rescaled(w, alpha, beta):
    """W~ = fp32(fp32(alpha_i * W_ij) * beta_j)."""
    w = np.asarray(w, np.float32)
    a = np.asarray(alpha, np.float32)[:, None]
    b = np.asarray(beta, np.float32)[None, :]
    return ((a * w).astype(np.float32) * b).astype(np.float32)


def qhat(w, alpha, beta, fmt):
    """fp64 values of Q(Diag(alpha) W Diag(beta)) (code x block scale, x t for NVFP4)."""
    codes, scales, t = quantize_rows(rescaled(w, alpha, beta), fmt)
    q = dequantize(pack_nibbles(codes), scales, fmt)
    return q * np.float64(t) if fmt == "nvfp4" else q


def axis_update(w, q, other, fmt, axis):
    """Projected inverse scales along `axis` (1: rows, r; 0: columns, c) for a
    fixed Q^ = q: each slice's 1-D least-squares coefficient of W against
    D = Q^ / (the other axis' scale, broadcast across the slice), projected
    to F; 1 where the slice of D is all zero."""
    other = np.asarray(other, np.float32).astype(np.float64)
    D = q / (other[None, :] if axis == 1 else other[:, None])
    wd = np.asarray(w, np.float32).astype(np.float64)
    num = exact_sums(wd * D, axis)
    den = exact_sums(D * D, axis)
    ok = den > 0
    return np.where(ok, project(num / np.where(ok, den, 1.0), fmt), 1.0)


def row_update(w, q, beta, fmt="mxfp4"):
    """Projected alpha^-1 (= r) from Q^ = q and the current beta."""
    return axis_update(w, q, beta, fmt, 1)


def col_update(w, q, alpha, fmt="mxfp4"):
    """Projected beta^-1 (= c) from Q^ = q and the current alpha."""
    return axis_update(w, q, alpha, fmt, 0)


def _inverse(x):
    x = np.asarray(x, np.float64)
    return np.where(x > 0, 1.0 / np.where(x > 0, x, 1.0), 1.0).astype(np.float32)


def init_scales(w):
    """alpha_0 = 1 / row absmax, beta_0 = 1 / column l1 norm (fp32)."""
    w = np.asarray(w, np.float32)
    amax = np.max(np.abs(w), axis=1).astype(np.float64)
    l1 = exact_sums(np.abs(w).astype(np.float64), 0)
    return _inverse(amax), _inverse(l1)


def mse(w, r, c, q):
    """|| W - Diag(r) Q^ Diag(c) ||_F^2 in fp64."""
    wd = np.asarray(w, np.float32).astype(np.float64)
    rec = np.asarray(r, np.float64)[:, None] * q * np.asarray(c, np.float64)[None, :]
    return float(np.sum((wd - rec) ** 2))


def half_step(w, alpha, beta, fmt, axis):
    """Synchronize Q^ with the current scales, then set the scales of one axis
    to their projected closed-form minimizers.  Returns (alpha, beta, inverse
    scales of that axis, Q^ used)."""
    q = qhat(w, alpha, beta, fmt)
    if axis == 1:
        r = axis_update(w, q, beta, fmt, 1)
        return (1.0 / r).astype(np.float32), beta, r, q
    c = axis_update(w, q, alpha, fmt, 0)
    return alpha, (1.0 / c).astype(np.float32), c, q


def solve(w, fmt, iters=15, history=None, stop_at_fixed_point=True):
    """Block coordinate descent on W (fp32 [N, K], K % 32 == 0).

    Returns (r fp32 [N], c fp32 [K], packed codes [N, K/2], scales [N, K/G],
    t_w fp32: the NVFP4 tensor scale of the final W~, 1 for MX).
    If `history` is a list, each half-step appends (axis, Q^, objective):
    axis "row" or "col", Q^ = Q(Diag(alpha) W Diag(beta)) re-quantized at the
    scales just set, and E there.
    """
    if fmt not in ("mxfp4", "mxint4", "nvfp4"):
        raise ValueError(f"unknown format {fmt}")
    w = np.asarray(w, np.float32)
    N, K = w.shape
    if K % 32 or iters < 1:
        raise ValueError("need K % 32 == 0 and iters >= 1")
    alpha, beta = init_scales(w)
    r = c = None
    for _ in range(iters):
        prev = (alpha, beta)
        for axis, name in ((1, "row"), (0, "col")):
            alpha, beta, s, _ = half_step(w, alpha, beta, fmt, axis)
            if axis == 1:
                r = s
            else:
                c = s
            if history is not None:
                q = qhat(w, alpha, beta, fmt)
                history.append((name, q, mse(w, 1.0 / alpha.astype(np.float64),
                                             1.0 / beta.astype(np.float64), q)))
        if stop_at_fixed_point and np.array_equal(prev[0], alpha) and np.array_equal(prev[1], beta):
            break              # a fixed point: the remaining iterations repeat this one
    codes, scales, t = quantize_rows(rescaled(w, alpha, beta), fmt)
    t_w = np.float32(t) if fmt == "nvfp4" else np.float32(1.0)
    return r.astype(np.float32), c.astype(np.float32), pack_nibbles(codes), scales, t_w
