"""Pins for the oracle's matvec, fused rows, argmax and small-batch product (CPU).

* one-hot x returns a column of the dequantised matrix bit-exactly;
* all-ones x over integer-valued blocks gives exact integer row sums;
* exact rational brute force (fractions) on tiny matrices;
* numpy float64 matmul of the dequantised matrix (a library routine);
* argmax against numpy's first-occurrence argmax, including planted ties;
* gemm_n: n = 1 equals the matvec, permuting X's rows permutes Y's rows.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import golden_blocks

TYPES = ["q8_0", "q4_k", "q6_k", "q4_0", "q4_1", "q5_0", "q5_1", "q8_1", "q5_k", "q2_k", "q3_k"]


def _matrix(t, M, K, seed):
    w = synth.weights(seed, M, K)
    return oracle.quantize(t, w)


@pytest.mark.parametrize("t", TYPES)
def test_one_hot_x_gives_column(t):
    M, K = 40, 512
    b = _matrix(t, M, K, 21)
    W = oracle.dequant(t, b, M, K)
    for k in [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 300, 511]:
        x = np.zeros(K, dtype=np.float32)
        x[k] = 1.0
        y, a = oracle.qmv(t, b, M, K, x)
        assert np.array_equal(y, W[:, k].astype(np.float64))
        assert np.array_equal(a, np.abs(W[:, k]).astype(np.float64))


def test_all_ones_integer_blocks_give_integer_row_sums():
    """Hand-built blocks have integer weights (d = dmin = 1), so the row sum
    with x = 1 is the exact integer sum of the hand-computed expectations."""
    for t, name, blk, expected in golden_blocks.load():
        if not all(v.denominator == 1 for v, _ in expected):
            continue
        n = len(expected)
        x = np.ones(n, dtype=np.float32)
        y, _ = oracle.qmv(t, blk, 1, n, x)
        assert y[0] == float(sum(v for v, _ in expected)), name


@pytest.mark.parametrize("t,K", [("q8_0", 64), ("q4_k", 256), ("q4_k", 512), ("q6_k", 256),
                                 ("q6_k", 512), ("q4_0", 64), ("q4_1", 64), ("q5_0", 64),
                                 ("q5_1", 64), ("q8_1", 64), ("q5_k", 256), ("q2_k", 256),
                                 ("q3_k", 512)])
def test_exact_rational_brute_force(t, K):
    M = 4
    b = _matrix(t, M, K, 22)
    x = synth.activations(23, K)
    W = oracle.dequant(t, b, M, K)
    y, a = oracle.qmv(t, b, M, K, x)
    for i in range(M):
        exact = sum(Fraction(float(W[i, k])) * Fraction(float(x[k])) for k in range(K))
        aex = sum(abs(Fraction(float(W[i, k])) * Fraction(float(x[k]))) for k in range(K))
        assert abs(Fraction(y[i]) - exact) <= Fraction(1, 10 ** 12) * aex
        assert abs(Fraction(a[i]) - aex) <= Fraction(1, 10 ** 12) * aex


@pytest.mark.parametrize("t", TYPES)
def test_matches_numpy_f64_matmul(t):
    M, K = 96, 2048
    b = _matrix(t, M, K, 24)
    x = synth.activations(25, K)
    W = oracle.dequant(t, b, M, K).astype(np.float64)
    y, a = oracle.qmv(t, b, M, K, x)
    ref = W @ x.astype(np.float64)
    aref = np.abs(W) @ np.abs(x.astype(np.float64))
    assert np.all(np.abs(y - ref) <= 1e-12 * aref)
    assert np.allclose(a, aref, rtol=1e-12, atol=0)


@pytest.mark.parametrize("t", TYPES)
def test_rows_subset_and_fused_segments(t):
    M, K = 48, 1024
    b = _matrix(t, M, K, 26)
    x = synth.activations(27, K)
    y, a = oracle.qmv(t, b, M, K, x)
    rows = np.array([47, 0, 13, 13, 30])
    ys, as_ = oracle.qmv_rows(t, b, M, K, x, rows)
    assert np.array_equal(ys, y[rows]) and np.array_equal(as_, a[rows])
    segs = oracle.fused_rows(t, b, K, x, [32, 8, 8])
    assert np.array_equal(np.concatenate([s[0] for s in segs]), y)


def test_argmax_matches_numpy_and_breaks_ties_low():
    t, M, K = "q6_k", 300, 512
    w = synth.weights(28, M, K)
    x = synth.activations(29, K)
    b = oracle.quantize(t, w)
    y, a = oracle.qmv(t, b, M, K, x)
    i, v, av = oracle.argmax(t, b, M, K, x)
    assert i == int(np.argmax(y)) and v == y[i] and av == a[i]
    # plant exact copies of the winning row at a higher and a lower index
    rb = oracle.row_bytes(t, K)
    b2 = b.copy()
    lo, hi = 5, 250
    for r in (lo, hi):
        b2[r * rb:(r + 1) * rb] = b[i * rb:(i + 1) * rb]
    y2, _ = oracle.qmv(t, b2, M, K, x)
    i2, v2, _ = oracle.argmax(t, b2, M, K, x)
    assert v2 == v and i2 == min(lo, i) == int(np.argmax(y2))


def test_argmax_planted_sign_row_wins():
    """A row proportional to sign(x) has the largest possible sum |x| among
    rows of its magnitude and wins by a wide margin."""
    t, M, K = "q8_0", 64, 256
    x = synth.activations(30, K)
    w = synth.weights(31, M, K)
    w[37] = 0.02 * np.sign(x)
    b = oracle.quantize(t, w)
    i, v, _ = oracle.argmax(t, b, M, K, x)
    assert i == 37
    y, _ = oracle.qmv(t, b, M, K, x)
    assert v - np.sort(y)[-2] > 0.5 * v


@pytest.mark.parametrize("t", ["q4_k", "q6_k"])
def test_gemm_n_columns(t):
    M, K = 32, 512
    b = _matrix(t, M, K, 32)
    X = synth.activations(33, K, n=8)
    Y, A = oracle.gemm_n(t, b, M, K, X)
    for j in range(8):
        y, a = oracle.qmv(t, b, M, K, X[j])
        assert np.array_equal(Y[j], y) and np.array_equal(A[j], a)
    perm = np.array([3, 1, 7, 0, 2, 6, 5, 4])
    Yp, _ = oracle.gemm_n(t, b, M, K, X[perm])
    assert np.array_equal(Yp, Y[perm])
