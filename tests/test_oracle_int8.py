"""Pins for the oracle's LLM.int8() (CPU only): the page's worked example, the
quantization steps against exact rational arithmetic, a lossless case where the
decomposition must reproduce X W^T exactly, and the page's central claim (the
decomposition removes the error an outlier column causes)."""

from fractions import Fraction

import numpy as np

from oracle import int8 as oi
from oracle.floats import fraction_to_f32


def test_page_example_column_17_is_the_outlier():
    """§2.1 【例子】: X (batch, hidden), threshold 6.0, X[:, 17] reaches 7.2 and every
    other column stays below 6.0: column 17 alone is cut out."""
    g = np.random.default_rng(1)
    X = np.clip(g.standard_normal((8, 64)), -5.9, 5.9).astype(np.float32)
    X[3, 17] = np.float32(7.2)
    out = oi.outlier_columns(X, 6.0)
    assert np.flatnonzero(out).tolist() == [17]
    assert not oi.outlier_columns(X, 0.0).any()           # threshold 0: no decomposition
    assert not oi.outlier_columns(X, 7.2).any()           # strictly greater


def test_row_quantization_matches_exact_arithmetic():
    g = np.random.default_rng(2)
    X = (g.standard_normal((5, 40)) * 3).astype(np.float32)
    X[2] = 0.0
    keep = np.ones(40, dtype=bool)
    keep[[3, 30]] = False
    q, a = oi.quantize_rows(X, keep)
    for r in range(5):
        amax = max(abs(float(X[r, k])) for k in range(40) if keep[k])
        assert a[r] == np.float32(amax)
        for k in range(40):
            if not keep[k] or amax == 0:
                assert q[r, k] == 0
                continue
            t = fraction_to_f32(Fraction(float(X[r, k])) / Fraction(amax))
            u = fraction_to_f32(Fraction(float(t)) * 127)
            fl = int(np.floor(float(u)))
            frac = Fraction(float(u)) - fl
            want = fl + (1 if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2) else 0)
            assert q[r, k] == want
    assert np.all(np.abs(q.astype(int)) <= 127)
    assert np.all(np.abs(q).max(axis=1)[a > 0] == 127)     # each row's extreme maps to +-127


def test_lossless_case_reproduces_the_product():
    """Values on the quantization grid: every row of W and of the kept part of X
    is RN(q * 2^e / 127) with a +-127 entry, so quantization gives back q and
    2^e; then the int8 path plus the outlier path equals the product of the grid
    values q * 2^e / 127 (and the outlier column as given)."""
    g = np.random.default_rng(3)
    M, N, K = 6, 7, 48
    CBt = g.integers(-127, 128, size=(N, K))
    CBt[:, 0] = 127
    sw = 2.0 ** g.integers(-3, 3, size=N)
    W = (CBt * sw[:, None] / 127).astype(np.float32)
    Xq = g.integers(-127, 128, size=(M, K))
    Xq[:, 1] = -127
    sx = 2.0 ** g.integers(-2, 2, size=M)
    X = (Xq * sx[:, None] / 127).astype(np.float32)
    X[:, 5] = np.float32(40.0)                            # an outlier column, off the grid
    CB, SCB = oi.quantize_rows(W)
    assert np.array_equal(CB.astype(int), CBt) and np.array_equal(SCB, sw.astype(np.float32))
    Y, out, Xq2, SX = oi.int8_matmul_f64(X, CB, SCB, 6.0)
    assert np.flatnonzero(out).tolist() == [5]
    keep = ~out
    assert np.array_equal(Xq2[:, keep].astype(int), Xq[:, keep]) and np.array_equal(SX, sx.astype(np.float32))
    # the grid values themselves (x = q s / 127 before any binary32 rounding), outlier column as given
    Xg = Xq * sx[:, None] / 127.0
    Xg[:, 5] = 40.0
    Wg = CBt * sw[:, None] / 127.0
    assert np.allclose(Y, Xg @ Wg.T, rtol=1e-12, atol=1e-12)


def test_decomposition_removes_the_outlier_error():
    """A column 50x larger than the rest: int8 alone (threshold 0) loses the
    small columns' precision; the decomposition keeps the error near the int8
    resolution."""
    g = np.random.default_rng(4)
    M, N, K = 64, 96, 512
    X = g.standard_normal((M, K)).astype(np.float32)
    X[:, 100] *= np.float32(50.0)
    W = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    CB, SCB = oi.quantize_rows(W)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    rel = lambda Y: np.linalg.norm(Y - exact) / np.linalg.norm(exact)
    y_mixed, out, _, _ = oi.int8_matmul_f64(X, CB, SCB, 6.0)
    y_int8, _, _, _ = oi.int8_matmul_f64(X, CB, SCB, 0.0)
    assert out[100] and out.sum() <= 3
    assert rel(y_mixed) < 0.02
    assert rel(y_int8) > 5 * rel(y_mixed)
