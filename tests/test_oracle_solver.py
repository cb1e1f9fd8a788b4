"""Pins of the oracle's DualQuant solver (Algorithm 1, MX formats) against
what the mathematics fixes: the projection against a brute-force search of
the admissible set, the closed-form updates against 1-D least squares and a
brute-force search of the projected objective (Appendix C, Remark 1), the
descent guarantee once Q^ has stabilized (Theorem 1), the degenerate-row
convention, the initialization, and exact power-of-two equivariance (MX).
For NVFP4 the admissible set is the positive E4M3 values."""
import numpy as np
import pytest

from oracle import solver as S

E8M0 = np.ldexp(1.0, np.arange(-127, 128))
# positive finite E4M3 values with their codes, from the bit layout
E4M3 = [(np.ldexp(float(m), -9) if e == 0 else np.ldexp(float(8 + m), e - 10), 8 * e + m)
        for e in range(16) for m in range(8) if 0 < 8 * e + m < 127]


def brute_nearest_e4m3(u):
    """argmin over the positive E4M3 values of |u - v|, ties to the even code."""
    out = []
    for x in np.asarray(u, np.float64):
        d = [(abs(v - x), code % 2, v) for v, code in E4M3]
        out.append(min(d)[2])
    return np.array(out)


def candidates(fmt):
    return np.array([v for v, _ in E4M3]) if fmt == "nvfp4" else E8M0


def brute(fmt, u):
    return brute_nearest_e4m3(u) if fmt == "nvfp4" else brute_nearest_e8m0(u)


def brute_nearest_e8m0(u):
    """argmin over all 255 powers of two of |u - 2^e|, ties to the larger."""
    out = []
    for x in np.asarray(u, np.float64):
        if x <= 0:
            out.append(E8M0[0])
            continue
        d = np.abs(E8M0 - x)
        best = np.flatnonzero(d == d.min())
        out.append(E8M0[best[-1]])
    return np.array(out)


def synthetic_weights(seed, N=64, K=256):
    rng = np.random.default_rng(seed)
    w = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    w[:, rng.choice(K, max(1, K // 64), replace=False)] *= 20
    w *= np.exp(rng.normal(0, 0.5, (1, K))).astype(np.float32)
    return w


def test_project_e8m0_matches_brute_force():
    rng = np.random.default_rng(0)
    u = np.ldexp(rng.uniform(0.5, 1.0, 4000), rng.integers(-140, 140, 4000))
    e = rng.integers(-126, 126, 200).astype(np.float64)
    mids = 1.5 * np.ldexp(1.0, e.astype(np.int64))
    special = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                              np.ldexp(1.0, e.astype(np.int64)), [0.0, -1.0, 1e-300, 1e300,
                                                                 2.0 ** 127, 1.5 * 2.0 ** 127]])
    x = np.concatenate([u, special])
    assert np.array_equal(S.project_e8m0(x), brute_nearest_e8m0(x))


def test_project_ue4m3_matches_brute_force():
    rng = np.random.default_rng(7)
    vals = np.array([v for v, _ in E4M3])
    mids = 0.5 * (vals[:-1] + vals[1:])
    x = np.concatenate([np.ldexp(rng.uniform(0.5, 1.0, 3000), rng.integers(-14, 11, 3000)),
                        mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf), vals,
                        [0.0, -2.0, 2.0 ** -11, 2.0 ** -10, 450.0, 480.0, 1e9]])
    assert np.array_equal(S.project_ue4m3(x), brute_nearest_e4m3(x))


def test_fixed_order_sums_are_sums():
    rng = np.random.default_rng(1)
    P = rng.normal(size=(70, 96))
    assert np.allclose(S.row_sums(P), P.sum(axis=1), rtol=1e-13, atol=1e-13)
    assert np.allclose(S.col_sums(P), P.sum(axis=0), rtol=1e-13, atol=1e-13)
    # the stated order, spelled out on one row and one column
    r = P[3].reshape(-1, 4, 8)
    blocks = [((sum8(b[0]) + sum8(b[1])) + sum8(b[2])) + sum8(b[3]) for b in r]
    acc = blocks[0]
    for v in blocks[1:]:
        acc = acc + v
    assert S.row_sums(P)[3] == acc
    col = P[:, 5]
    c0 = sum_seq(col[:16])
    assert S.col_sums(P)[5] == (((c0 + sum_seq(col[16:32])) + sum_seq(col[32:48])) + sum_seq(col[48:64])) + sum_seq(col[64:])


def sum8(v):
    return sum_seq(v)


def sum_seq(v):
    acc = v[0]
    for x in v[1:]:
        acc = acc + x
    return acc


@pytest.mark.parametrize("fmt", ["mxfp4", "mxint4", "nvfp4"])
def test_row_update_is_projected_least_squares(fmt):
    """For fixed Q^ and beta, the row scale minimizes the row's squared error
    over the admissible set: the unconstrained minimizer is the 1-D least
    squares coefficient and its nearest power of two is the constrained one."""
    w = synthetic_weights(2, N=24, K=128)
    rng = np.random.default_rng(3)
    alpha = np.ldexp(1.0, rng.integers(-2, 3, 24)).astype(np.float32) * np.float32(7.3)
    beta = np.exp(rng.normal(0, 0.7, 128)).astype(np.float32)
    q = S.qhat(w, alpha, beta, fmt)
    r = S.row_update(w, q, beta, fmt)
    R = q / beta.astype(np.float64)[None, :]
    wd = w.astype(np.float64)
    for i in range(24):
        if not np.any(R[i]):
            assert r[i] == 1.0
            continue
        ls = np.linalg.lstsq(R[i][:, None], wd[i], rcond=None)[0][0]
        assert np.isclose(ls, np.dot(wd[i], R[i]) / np.dot(R[i], R[i]), rtol=1e-12)
        assert r[i] == brute(fmt, [ls])[0]
        err = [np.sum((wd[i] - v * R[i]) ** 2) for v in candidates(fmt)]
        assert np.sum((wd[i] - r[i] * R[i]) ** 2) <= min(err) * (1 + 1e-12)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxint4", "nvfp4"])
def test_col_update_is_projected_least_squares(fmt):
    w = synthetic_weights(4, N=40, K=64)
    rng = np.random.default_rng(5)
    alpha = np.exp(rng.normal(0, 0.5, 40)).astype(np.float32)
    beta = np.ldexp(1.0, rng.integers(-3, 3, 64)).astype(np.float32)
    q = S.qhat(w, alpha, beta, fmt)
    c = S.col_update(w, q, alpha, fmt)
    Sm = q / alpha.astype(np.float64)[:, None]
    wd = w.astype(np.float64)
    for j in range(64):
        if not np.any(Sm[:, j]):
            assert c[j] == 1.0
            continue
        ls = np.dot(wd[:, j], Sm[:, j]) / np.dot(Sm[:, j], Sm[:, j])
        assert c[j] == brute(fmt, [ls])[0]
        err = [np.sum((wd[:, j] - v * Sm[:, j]) ** 2) for v in candidates(fmt)]
        assert np.sum((wd[:, j] - c[j] * Sm[:, j]) ** 2) <= min(err) * (1 + 1e-12)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxint4"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_descent_after_stabilization(fmt, seed):
    """Theorem 1 (i): once Q^ no longer changes, every half-step keeps or
    lowers the objective.  (MX only: with NVFP4 the tensor scale of W~ moves
    with every rescaling, so Q^ need not stabilize.)"""
    w = synthetic_weights(10 + seed)
    hist = []
    S.solve(w, fmt, 6, hist)
    stable = next(i for i in range(1, len(hist)) if np.array_equal(hist[i][1], hist[i - 1][1]))
    objs = [h[2] for h in hist]
    for i in range(stable, len(objs) - 1):
        assert objs[i + 1] <= objs[i] * (1 + 1e-12)


def test_degenerate_rows_and_columns():
    w = synthetic_weights(20)
    w[5] = 0
    w[:, 7] = 0
    for fmt in ("mxfp4", "mxint4", "nvfp4"):
        r, c, codes, scales, _ = S.solve(w, fmt, 3)
        assert r[5] == 1.0 and c[7] == 1.0
        assert not np.any(codes[5]) and scales[5].max() == 0


def test_init_is_inverse_absmax_and_l1():
    w = synthetic_weights(21)
    alpha, beta = S.init_scales(w)
    assert np.array_equal(alpha, (1.0 / np.abs(w).max(axis=1).astype(np.float64)).astype(np.float32))
    l1 = np.abs(w).astype(np.float64).sum(axis=0)
    assert np.allclose(beta, (1.0 / l1).astype(np.float32), rtol=2 ** -23)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxint4"])
def test_power_of_two_equivariance(fmt):
    """W -> 2^k W scales the initial scales by 2^-k exactly and the MX
    quantizer is equivariant under powers of two, so r and c scale by 2^k and
    the codes stay the same (the reconstruction scales by 2^k)."""
    w = synthetic_weights(22)
    r, c, codes, scales, _ = S.solve(w, fmt, 4)
    r2, c2, codes2, scales2, _ = S.solve(np.ldexp(w, 3).astype(np.float32), fmt, 4)
    assert np.array_equal(r2, np.ldexp(r, 3)) and np.array_equal(c2, np.ldexp(c, 3))
    assert np.array_equal(codes2, codes)
    assert np.array_equal(scales2.astype(int), scales.astype(int) - 3)
