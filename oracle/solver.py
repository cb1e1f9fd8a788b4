"""DualQuant's offline dual-scale solver (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed: Algorithm 1 of the pages ("DualQuant: Dual-Scale
Quantization via Coordinate Descent", Section 4.3 "MSE optimization via block
coordinate descent"), which minimizes the weight-reconstruction error

    || W - Diag(alpha)^-1 Q(Diag(alpha) W Diag(beta)) Diag(beta)^-1 ||_F^2

over a row scale alpha (one per output row) and a column scale beta (one per
input column) whose inverses live in the format's admissible set F (Section
4.2; E8M0 for the MX formats, UE4M3 for NVFP4).  Q is the format's row-wise
block quantizer (Section 3; `quant.quantize_rows`; for NVFP4 with the fp32
tensor scale of the tensor it quantizes).  Each iteration:

  1. Q^ = Q(Diag(alpha) W Diag(beta)); R = Q^ Diag(beta)^-1;
     alpha^-1_i = Pi_F( <W_i, R_i> / ||R_i||^2 ), the closed-form minimizer
     of the row's 1-D quadratic (Section 4.3, "Closed-form scale updates"),
     projected to the nearest admissible value (Appendix C, Remark 1);
  2. Q^ = Q(Diag(alpha) W Diag(beta)) with the new alpha; S = Diag(alpha)^-1 Q^;
     beta^-1_j = Pi_F( <W_j, S_j> / ||S_j||^2 ) over the column.

It returns r = alpha^-1, c = beta^-1 and Q(Diag(alpha) W Diag(beta)), so that
W ~ Diag(r) Q Diag(c): r goes into the packed weight, c into the activation
quantizer.  Initialization (Section 5, "Hyperparameter selection"): the
row absmax and the column l1 norm; T = 15 by default.

Readings where the pages leave a step open:
  * Initialization: alpha_0,i^-1 = max_j |W_ij| and beta_0,j^-1 = sum_i |W_ij|,
    i.e. the inverse scales start at those magnitudes (the extracted text
    shows the magnitudes without an inverse marker).  Taken literally (alpha_0
    = absmax) the solver ends about 2x above round-to-nearest on synthetic
    weights with outlier columns; with the inverse it ends 1.3-1.9x below
    (MX formats), and beta then follows a weight-only smoothing scale, as the pages report.
    alpha_0 = fp32(1 / absmax) and beta_0 = fp32(1 / l1) from fp64 quotients;
    an all-zero row or column starts at 1.
  * The rescaled weight is W~_ij = fp32(fp32(alpha_i * W_ij) * beta_j), with
    alpha = fp32(1 / r) and beta = fp32(1 / c) (fp64 quotients rounded to
    fp32; exact for E8M0) and fp32 W.  For NVFP4, Q^ includes the tensor
    scale t of W~ (code x block scale x t, exact in fp64), and the returned
    codes come with the t of the final W~ (t_w; 1 for the MX formats).
  * Q^, R and S are fp64 values (Q^ = code x block scale is exact; R and S
    one fp64 division each); the inner products and squared norms are fp64
    sums taken in a fixed order, so that another implementation following
    the same order reaches the same projected scales:
      rows:    8 consecutive terms sequentially, the four such partials of a
               32-block as ((p0 + p1) + p2) + p3, then the blocks in order;
      columns: rows in chunks of 16, each chunk sequentially, then the chunks
               in order.
    beta_0 uses the column order; alpha_0 is an exact maximum.
  * The projection is to the nearest admissible value in linear distance
    (Remark 1: the subproblem is a convex quadratic in the inverse scale).
    E8M0: the powers of two 2^e, e in [-127, 127]; an exact tie 1.5 * 2^e
    goes to 2^(e+1); a non-positive minimizer goes to 2^-127.  UE4M3: the
    126 positive finite E4M3 values (zero would zero the row); ties go to
    the even code, as in E4M3 rounding; above 448 saturates; a minimizer
    below 2^-9 (or non-positive) goes to 2^-9.
  * A row (column) whose Q^ is all zero has no minimizer; its scale is set to
    1 (the pages' convention for rows, applied to columns alike).
"""
from __future__ import annotations

import numpy as np

from .quant import quantize_rows, pack_nibbles, dequantize

E8M0_MIN = 2.0 ** -127
E8M0_MAX = 2.0 ** 127
COL_CHUNK = 16


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


def row_sums(P):
    """Sum of each row of P [N, K] (K % 32 == 0) in the fixed order above."""
    P = np.asarray(P, np.float64)
    N, K = P.shape
    q = P.reshape(N, K // 32, 4, 8)
    p = q[..., 0].copy()
    for t in range(1, 8):
        p = p + q[..., t]
    b = ((p[..., 0] + p[..., 1]) + p[..., 2]) + p[..., 3]
    s = b[:, 0].copy()
    for j in range(1, K // 32):
        s = s + b[:, j]
    return s


def col_sums(P):
    """Sum of each column of P [N, K] in the fixed order above."""
    P = np.asarray(P, np.float64)
    N, K = P.shape
    total = None
    for r0 in range(0, N, COL_CHUNK):
        blk = P[r0:r0 + COL_CHUNK]
        s = blk[0].copy()
        for i in range(1, blk.shape[0]):
            s = s + blk[i]
        total = s if total is None else total + s
    return total


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


def _update(num, den, fmt):
    ok = den > 0
    return np.where(ok, project(num / np.where(ok, den, 1.0), fmt), 1.0)


def row_update(w, q, beta, fmt="mxfp4"):
    """Projected alpha^-1 (= r) from Q^ = q and the current beta."""
    R = q / np.asarray(beta, np.float32).astype(np.float64)[None, :]
    wd = np.asarray(w, np.float32).astype(np.float64)
    return _update(row_sums(wd * R), row_sums(R * R), fmt)


def col_update(w, q, alpha, fmt="mxfp4"):
    """Projected beta^-1 (= c) from Q^ = q and the current alpha."""
    S = q / np.asarray(alpha, np.float32).astype(np.float64)[:, None]
    wd = np.asarray(w, np.float32).astype(np.float64)
    return _update(col_sums(wd * S), col_sums(S * S), fmt)


def _inverse(x):
    x = np.asarray(x, np.float64)
    return np.where(x > 0, 1.0 / np.where(x > 0, x, 1.0), 1.0).astype(np.float32)


def init_scales(w):
    """alpha_0 = 1 / row absmax, beta_0 = 1 / column l1 norm (fp32)."""
    w = np.asarray(w, np.float32)
    amax = np.max(np.abs(w), axis=1).astype(np.float64)
    l1 = col_sums(np.abs(w).astype(np.float64))
    return _inverse(amax), _inverse(l1)


def mse(w, r, c, q):
    """|| W - Diag(r) Q^ Diag(c) ||_F^2 in fp64."""
    wd = np.asarray(w, np.float32).astype(np.float64)
    rec = np.asarray(r, np.float64)[:, None] * q * np.asarray(c, np.float64)[None, :]
    return float(np.sum((wd - rec) ** 2))


def solve(w, fmt, iters=15, history=None):
    """Algorithm 1 on W (fp32 [N, K], K % 32 == 0).

    Returns (r fp32 [N], c fp32 [K], packed codes [N, K/2], scales [N, K/G],
    t_w fp32: the NVFP4 tensor scale of the final W~, 1 for MX).
    If `history` is a list, each half-step appends (phase, Q^, objective):
    phase "row" or "col", Q^ = Q(Diag(alpha) W Diag(beta)) at the scales just
    updated and the objective || W - Diag(alpha)^-1 Q^ Diag(beta)^-1 ||^2 there.
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
        q = qhat(w, alpha, beta, fmt)
        r = row_update(w, q, beta, fmt)
        alpha = (1.0 / r).astype(np.float32)
        q = qhat(w, alpha, beta, fmt)
        if history is not None:
            history.append(("row", q, mse(w, 1.0 / alpha.astype(np.float64),
                                          1.0 / beta.astype(np.float64), q)))
        c = col_update(w, q, alpha, fmt)
        beta = (1.0 / c).astype(np.float32)
        if history is not None:
            qn = qhat(w, alpha, beta, fmt)
            history.append(("col", qn, mse(w, r, c, qn)))
    codes, scales, t = quantize_rows(rescaled(w, alpha, beta), fmt)
    t_w = np.float32(t) if fmt == "nvfp4" else np.float32(1.0)
    return r.astype(np.float32), c.astype(np.float32), pack_nibbles(codes), scales, t_w
