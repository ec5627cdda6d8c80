"""GPU parity for qmv_gemm, the prefill-size product Y[n][M] = X[n][K] W^T
(BebeLM page, section "性能表现": prompt tokens go through as a batch),
against the oracle's f64 product (the same definition as the small batch).

Bound: as the verify product (exact codes on the matrix cores, X as bf16
hi + lo, f32 scales), within 1e-5 * sum_k |w_ik X[j][k]| per output.
Also: permuting X's rows permutes Y's rows bit for bit (tokens are
independent MFMA rows) and two runs are identical (K slices, when there
are several, are added in a fixed order).
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
    wsb = q.qmv_workspace_bytes(q.OP_GEMM, M, K, n)
    ws = empty(wsb, "uint8") if wsb else None
    q.qmv_gemm(t, bd, M, K, n, dev(X), Y, ws)
    return host(Y).reshape(n, M)


SHAPES = [
    ("q4_k", 300, 4096, 100),    # ragged rows and a partial token block
    ("q4_k", 129, 2048, 64),
    ("q4_k", 40, 256, 17),
    ("q6_k", 129, 1536, 70),
    ("q6_k", 64, 4096, 33),
    ("q8_0", 77, 224, 130),      # a partial last window of Q8_0 blocks
    ("q8_0", 200, 576, 65),
    ("q4_k", 33, 512, 1),
    # few rows and tokens, long K: K split into slices
    ("q4_k", 300, 14336, 20),
    ("q6_k", 129, 4096, 70),
    ("q8_0", 200, 4000, 40),     # slices, the last one ending in a partial window
    ("q4_k", 1000, 4096, 16),
    ("q5_k", 300, 4096, 100),    # Q5_K: the Q4_K policy plus fifth bits
    ("q5_k", 129, 14336, 20),    # and with K slices
    # one workgroup per compute unit with several 16-row tiles per wave:
    ("q4_k", 2048, 256, 4096),   # four row tiles, four token tiles (512-row workgroups)
    ("q5_k", 2100, 512, 4000),   # the same with a ragged row group and token block
    ("q4_k", 3000, 256, 1000),   # two row tiles, four token tiles
    ("q4_k", 4000, 512, 500),    # two row tiles, two token tiles
    ("q6_k", 1100, 1024, 1000),  # planned with four row tiles: Q6_K runs two, twice the groups
    ("q8_0", 2100, 544, 1500),   # the same for Q8_0, ending in a partial window
]


@pytest.mark.parametrize("t,M,K,n", SHAPES)
def test_gemm_parity(t, M, K, n):
    b = quantized(t, M, K, 1100 + M)
    X = synth.activations(1101 + M, K, n=n)
    Yr, Ar = oracle.gemm_n(t, b, M, K, X)
    Y = gemm_gpu(t, dev(b), M, K, X)
    worst = assert_rel(Y.ravel(), Yr.ravel(), Ar.ravel(), what=f"{t} {M}x{K} n={n}")
    print(f"{t} {M}x{K} n={n}: worst |dY|/sum|wx| = {worst:.2e}")


@pytest.mark.parametrize("t", ["q4_k", "q5_k", "q6_k", "q8_0"])
def test_gemm_token_permutation_and_determinism(t):
    M, K, n = 260, 1024, 150
    b = quantized(t, M, K, 1110)
    X = synth.activations(1111, K, n=n)
    bd = dev(b)
    Y = gemm_gpu(t, bd, M, K, X)
    perm = np.random.default_rng(7).permutation(n)
    Yp = gemm_gpu(t, bd, M, K, X[perm])
    assert np.array_equal(Yp.view(np.uint32), Y[perm].view(np.uint32))
    Y2 = gemm_gpu(t, bd, M, K, X)
    assert np.array_equal(Y2.view(np.uint32), Y.view(np.uint32))


def test_gemm_llama8b_gate_up_n512_sampled():
    t, M, K, n = "q4_k", sum(synth.CONFIG4["gate_up"]), synth.CONFIG4["hidden"], 512
    b = quantized(t, M, K, 902)
    X = synth.activations(1120, K, n=n)
    Y = gemm_gpu(t, dev(b), M, K, X)
    g = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, M - 1], g.integers(0, M, 48)])).astype(np.int64)
    for j in [0, 1, 63, 64, 200, 511]:
        yr, ar = oracle.qmv_rows(t, b, M, K, X[j], rows)
        assert_rel(Y[j, rows], yr, ar, what=f"token {j}")


@pytest.mark.parametrize("n", [256, 512])
def test_gemm_llama8b_down_sampled(n):
    """The 4096 x 14336 down projection as the 32-layer prefill pass runs it:
    K split into four slices, with one row tile per wave at n = 256 and two
    at n = 512 (long slices), checked on sampled rows of sampled tokens."""
    t, (M, K) = "q4_k", synth.CONFIG4["down"]
    wsb = q.qmv_workspace_bytes(q.OP_GEMM, M, K, n)
    assert wsb - (n // 16) * (K // 256) * 1088 * 16 == 4 * 4 * n * M
    b = quantized(t, M, K, 903)
    X = synth.activations(1125 + n, K, n=n)
    Y = gemm_gpu(t, dev(b), M, K, X)
    g = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, M - 1], g.integers(0, M, 40)])).astype(np.int64)
    for j in [0, 1, 63, 64, 129, n - 1]:
        yr, ar = oracle.qmv_rows(t, b, M, K, X[j], rows)
        assert_rel(Y[j, rows], yr, ar, what=f"down n={n} token {j}")


@pytest.mark.parametrize("t", ["q4_k", "q5_k"])
def test_gemm_two_tiles_with_k_slices(t):
    """Few 256-row groups, six 64-token blocks and long K: two row tiles per
    wave with K in eight slices of twelve windows (a ragged last row group
    and token block), every token on sampled rows."""
    M, K, n = 1100, 24576, 330
    wsb = q.qmv_workspace_bytes(q.OP_GEMM, M, K, n)
    assert wsb - 6 * 64 * (K // 256) * 1088 == -(-(8 * 4 * n * M) // 256) * 256
    b = quantized(t, M, K, 1140)
    X = synth.activations(1141, K, n=n)
    Y = gemm_gpu(t, dev(b), M, K, X)
    g = np.random.default_rng(12)
    rows = np.unique(np.concatenate([[0, 255, 256, 1023, 1024, M - 1],
                                     g.integers(0, M, 24)])).astype(np.int64)
    for j in range(n):
        yr, ar = oracle.qmv_rows(t, b, M, K, X[j], rows)
        assert_rel(Y[j, rows], yr, ar, what=f"{t} token {j}")


@pytest.mark.parametrize("t,M,K,n", [("q4_k", 300, 4096, 70), ("q6_k", 129, 1536, 40),
                                     ("q8_0", 77, 576, 33), ("q5_k", 129, 14336, 20)])
def test_gemm_wide_range_x(t, M, K, n):
    """Tokens whose scales differ by up to 1e40, values within a token over
    1e6, and an all-zero token: the bf16 hi + lo split made once per call
    keeps every output within the bound (no overflow, no lost small token)."""
    b = quantized(t, M, K, 840 + n)
    g = np.random.default_rng(841 + n)
    X = g.standard_normal((n, K)) * 10.0 ** g.integers(-3, 3, (n, K))
    X *= 10.0 ** g.integers(-20, 20, (n, 1))
    X[n // 2] = 0.0
    X = X.astype(np.float32)
    Yr, Ar = oracle.gemm_n(t, b, M, K, X)
    Y = gemm_gpu(t, dev(b), M, K, X)
    assert np.all(Y[n // 2] == 0.0)
    assert_rel(Y.ravel(), Yr.ravel(), Ar.ravel(), what="wide-range X")


def test_gemm_split_k_is_deterministic_and_within_bound():
    """A K-split call (few rows and tokens) is deterministic and agrees with
    the oracle; its workspace is a whole number of n x M f32 slices plus the
    staged activations (1088 bytes per 16 tokens and 256 values; n = 32
    fills its token blocks exactly)."""
    t, M, K, n = "q4_k", 256, 14336, 32
    wsb = q.qmv_workspace_bytes(q.OP_GEMM, M, K, n)
    rest = wsb - (-(-n // 16)) * (-(-K // 256)) * 1088 * 16
    assert rest > 0 and rest % (4 * n * M) == 0 and 2 <= rest // (4 * n * M) <= 16
    b = quantized(t, M, K, 1130)
    X = synth.activations(1131, K, n=n)
    bd = dev(b)
    Y = gemm_gpu(t, bd, M, K, X)
    Y2 = gemm_gpu(t, bd, M, K, X)
    assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32))
    Yr, Ar = oracle.gemm_n(t, b, M, K, X)
    assert_rel(Y.ravel(), Yr.ravel(), Ar.ravel(), what="split K")
