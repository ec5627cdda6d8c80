"""GPU parity for qmv_gemm_n (small-batch verify on the matrix cores) against
the oracle's f64 Y[j][i] = sum_k w_ik X[j][k].

Bound: the MFMA sees the exact integer codes and X split into bf16 hi + lo,
so the representation error is <= 2^-18 |x| per product, plus f32
accumulation: within the matvec's 1e-5 * sum_k |w_ik X[j][k]| per output.
Also: n = 1 matches the matvec within the bound; permuting X's rows permutes
Y's rows bit for bit (each token is an independent MFMA row); two runs are
identical (the waves' and the K slices' partial sums are added in a fixed
order).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_rel, dev, empty, host, quantized

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gguf_dequant_matvec_amd as q  # noqa: E402


def gemm_gpu(t, bd, M, K, X):
    n = X.shape[0]
    Y = empty(n * M)
    ws_n = q.qmv_workspace_bytes(q.OP_GEMM_N, M, K, n)
    ws = empty(max(ws_n, 16), "uint8")
    q.qmv_gemm_n(t, bd, M, K, n, dev(X), Y, ws)
    return host(Y).reshape(n, M)


SHAPES = [
    ("q4_k", 300, 4096, 8), ("q4_k", 129, 2048, 16), ("q4_k", 64, 256, 16),
    ("q4_k", 1000, 14336, 16), ("q4_k", 4096, 4096, 16),
    ("q6_k", 200, 1536, 16), ("q6_k", 77, 4096, 3), ("q6_k", 500, 4096, 8),
    ("q8_0", 100, 576, 16), ("q8_0", 37, 224, 5), ("q8_0", 300, 4096, 16), ("q8_0", 17, 32, 2),
    ("q5_k", 300, 4096, 16), ("q5_k", 129, 2048, 7), ("q5_k", 1000, 14336, 16),
    ("q4_k", 50, 4096, 1), ("q4_k", 333, 4096, 9), ("q6_k", 64, 1536, 1), ("q8_0", 70, 4096, 8),
]


@pytest.mark.parametrize("t,M,K,n", SHAPES)
def test_gemm_n_parity(t, M, K, n):
    b = quantized(t, M, K, 800 + M)
    X = synth.activations(801 + M, K, n=n)
    Yr, Ar = oracle.gemm_n(t, b, M, K, X)
    Y = gemm_gpu(t, dev(b), M, K, X)
    worst = assert_rel(Y.ravel(), Yr.ravel(), Ar.ravel(), what=f"{t} {M}x{K} n={n}")
    print(f"{t} {M}x{K} n={n}: worst |dY|/sum|wx| = {worst:.2e}")


def test_gemm_n_one_column_matches_matvec():
    t, M, K = "q4_k", 777, 4096
    b = quantized(t, M, K, 810)
    x = synth.activations(811, K)
    bd = dev(b)
    Y = gemm_gpu(t, bd, M, K, x[None, :])
    y = empty(M)
    q.qmv(t, bd, M, K, dev(x), y)
    yr, ar = oracle.qmv(t, b, M, K, x)
    assert_rel(Y[0], yr, ar)
    assert np.all(np.abs(Y[0].astype(np.float64) - host(y)) <= 2e-5 * ar)


@pytest.mark.parametrize("t", ["q4_k", "q5_k", "q6_k", "q8_0"])
def test_gemm_n_token_permutation_and_determinism(t):
    M, K = 333, 4096
    b = quantized(t, M, K, 820)
    bd = dev(b)
    for n in (16, 8):             # both operand layouts
        X = synth.activations(821 + n, K, n=n)
        Y = gemm_gpu(t, bd, M, K, X)
        perm = np.random.default_rng(5).permutation(n)
        Yp = gemm_gpu(t, bd, M, K, X[perm])
        assert np.array_equal(Yp.view(np.uint32), Y[perm].view(np.uint32)), n
        Y2 = gemm_gpu(t, bd, M, K, X)
        assert np.array_equal(Y2.view(np.uint32), Y.view(np.uint32)), n


def test_gemm_n_wide_range_x():
    t, M, K, n = "q6_k", 128, 4096, 16
    b = quantized(t, M, K, 830)
    g = np.random.default_rng(831)
    X = (g.standard_normal((n, K)) * 10.0 ** g.integers(-6, 6, (n, K))).astype(np.float32)
    Yr, Ar = oracle.gemm_n(t, b, M, K, X)
    Y = gemm_gpu(t, dev(b), M, K, X)
    assert_rel(Y.ravel(), Yr.ravel(), Ar.ravel(), what="wide-range X")


# Shapes that take each part of the launch plan (windows of 256 weights;
# waves per tile along K = the largest power of two <= the windows, at most
# 8; one or two windows per wave; K slices only past 16 windows): one window
# (ks = 1, eight tiles per group), 5 windows (ks = 4), 9 windows (one wave
# with two, seven with one), 16 windows (ks = 8, many tiles per workgroup,
# batches of four), a Q8_0 row whose last window holds one block and that
# splits into two K slices, a Q8_0 row of 23 blocks, n = 9 (the first n of
# the two-MFMA layout) and ragged row counts.  Checked on sampled rows, and
# repeated runs are bit-identical.
SHAPES_PLAN = [
    ("q4_k", 16384, 4096, 16), ("q4_k", 65536 + 77, 256, 8), ("q4_k", 16384 + 5, 2304, 3),
    ("q6_k", 8192, 4096, 8), ("q5_k", 8192 + 100, 4096, 16), ("q8_0", 8192, 4128, 16),
    ("q4_k", 2000 + 3, 1280, 9), ("q8_0", 3000 + 1, 736, 4), ("q6_k", 1000, 6144, 12),
]


def sampled_rows(M, seed, n=300):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, M // 2, M - 2, M - 1], g.integers(0, M, n)]))


@pytest.mark.parametrize("t,M,K,n", SHAPES_PLAN)
def test_gemm_n_launch_plans(t, M, K, n):
    b = quantized(t, M, K, 840 + K)
    X = synth.activations(841 + K, K, n=n)
    bd = dev(b)
    Y = gemm_gpu(t, bd, M, K, X)
    rows = sampled_rows(M, 842 + K)
    rb = q.row_bytes(t, K)
    bs = b.reshape(M, rb)[rows].ravel()
    Yr, Ar = oracle.gemm_n(t, bs, len(rows), K, X)
    worst = assert_rel(Y[:, rows].ravel(), Yr.ravel(), Ar.ravel(), what=f"{t} {M}x{K} n={n}")
    print(f"{t} {M}x{K} n={n} ({len(rows)} sampled rows): worst {worst:.2e}")
    Y2 = gemm_gpu(t, bd, M, K, X)
    assert np.array_equal(Y2.view(np.uint32), Y.view(np.uint32))
