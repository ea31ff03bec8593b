"""Pins for the oracle's GEMV / GEMM arithmetic (CPU only).

- brute force in exact rationals (fractions.Fraction) on 1x32 and 4x256
  matrices: the oracle's fp64 result must lie within k * 2^-53 * sum|w x|;
- closed forms: x = e_k selects column k of W; x = 0 gives 0;
- invariants: each batch column equals the batch-1 result; each GEMM row
  equals the GEMV of that row converted to fp32; sum|w x| is the sum of
  absolute products.
The exact weight values come from ``dequant_f64``, itself pinned by
test_oracle_decode.py.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import qmm_inputs
import packing as P

TYPES = [P.Q4_0, P.Q8_0, P.Q4_K, P.Q6_K, P.Q5_0, P.Q5_K]


def _exact_dot(wrow, xrow):
    s = Fraction(0)
    sa = Fraction(0)
    for a, b in zip(wrow, xrow):
        p = Fraction(float(a)) * Fraction(float(b))
        s += p
        sa += abs(p)
    return s, sa


@pytest.mark.parametrize("t,n,k", [(P.Q8_0, 1, 32), (P.Q4_0, 1, 32), (P.Q5_0, 1, 32)] + [(t, 4, 256) for t in TYPES])
def test_gemv_exact_rationals(t, n, k):
    w = qmm_inputs.gen_weights(t, n, k, seed=21 + t)
    x = qmm_inputs.gen_x(k, 2, seed=22 + t)
    wexact = oracle.dequant_f64(t, w, n, k)
    w32 = oracle.dequant(t, w, n, k)
    assert np.array_equal(wexact.astype(np.float32), w32)
    y, a = oracle.gemv(t, w, n, k, x)
    for b in range(2):
        for r in range(n):
            s, sa = _exact_dot(w32[r], x[b])
            assert abs(Fraction(y[b, r]) - s) <= Fraction(k) * Fraction(2) ** -53 * sa
            assert abs(Fraction(a[b, r]) - sa) <= Fraction(k) * Fraction(2) ** -53 * sa


@pytest.mark.parametrize("t", TYPES)
def test_gemm_exact_rationals(t):
    n, k, m = 3, 256, 3
    w = qmm_inputs.gen_weights(t, n, k, seed=31 + t)
    X = qmm_inputs.gen_x_f16(m, k, seed=32 + t)
    w32 = oracle.dequant(t, w, n, k)
    Y, A = oracle.gemm(t, w, n, k, X)
    for i in range(m):
        for r in range(n):
            s, sa = _exact_dot(w32[r], X[i].astype(np.float64))
            assert abs(Fraction(Y[i, r]) - s) <= Fraction(k) * Fraction(2) ** -53 * sa


@pytest.mark.parametrize("t", TYPES)
def test_gemv_one_hot_selects_column(t):
    n, k = 5, 512
    w = qmm_inputs.gen_weights(t, n, k, seed=41 + t)
    w32 = oracle.dequant(t, w, n, k)
    for col in (0, 1, 31, 32, 255, 256, 511):
        x = np.zeros((1, k), np.float32)
        x[0, col] = 1.0
        y, a = oracle.gemv(t, w, n, k, x)
        assert np.array_equal(y[0], w32[:, col].astype(np.float64))
        assert np.array_equal(a[0], np.abs(w32[:, col]).astype(np.float64))
    y, a = oracle.gemv(t, w, n, k, np.zeros((1, k), np.float32))
    assert not y.any() and not a.any()


@pytest.mark.parametrize("t", TYPES)
def test_gemv_batch_columns_and_gemm_rows(t):
    n, k = 7, 512
    w = qmm_inputs.gen_weights(t, n, k, seed=51 + t)
    x = qmm_inputs.gen_x(k, 8, seed=52 + t)
    y, a = oracle.gemv(t, w, n, k, x)
    for b in range(8):
        y1, a1 = oracle.gemv(t, w, n, k, x[b:b + 1])
        assert np.array_equal(y1[0], y[b]) and np.array_equal(a1[0], a[b])
    X = qmm_inputs.gen_x_f16(6, k, seed=53 + t)
    Y, A = oracle.gemm(t, w, n, k, X)
    yv, av = oracle.gemv(t, w, n, k, X.astype(np.float32))
    assert np.array_equal(Y, yv) and np.array_equal(A, av)
    Ys, As = oracle.gemm(t, w, n, k, X, rows=[5, 0, 3])
    assert np.array_equal(Ys, Y[[5, 0, 3]]) and np.array_equal(As, A[[5, 0, 3]])


@pytest.mark.parametrize("t", TYPES)
def test_abs_sum_and_orientation(t):
    """sum|w x| against numpy on the dequantized matrix, and y = W x (not
    W^T x): a transposed operand fails the non-square case."""
    n, k = 3, 2 * P.BE[t]
    w = qmm_inputs.gen_weights(t, n, k, seed=61 + t)
    x = qmm_inputs.gen_x(k, 1, seed=62 + t)
    w32 = oracle.dequant(t, w, n, k).astype(np.float64)
    y, a = oracle.gemv(t, w, n, k, x)
    assert np.allclose(y[0], w32 @ x[0].astype(np.float64), rtol=1e-12, atol=0)
    assert np.allclose(a[0], np.abs(w32) @ np.abs(x[0].astype(np.float64)), rtol=1e-12, atol=0)


def test_empty_shapes():
    w = np.zeros(0, np.uint8)
    y, a = oracle.gemv(P.Q8_0, w, 0, 64, np.zeros((1, 64), np.float32))
    assert y.shape == (1, 0)
    w = qmm_inputs.gen_weights(P.Q8_0, 3, 32, seed=1)[:, :0].copy()
    y, a = oracle.gemv(P.Q8_0, np.zeros(0, np.uint8), 3, 0, np.zeros((2, 0), np.float32))
    assert y.shape == (2, 3) and not y.any()
