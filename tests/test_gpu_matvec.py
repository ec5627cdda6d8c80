"""GPU parity: dequantisation, single-token matvec, fused rows, argmax and the
quantiser of libqmv against the CPU oracle, through the C ABI.

Bars: dequantised values and argmax indices bit-exact; matvec outputs within
1e-5 * sum_k |w_ik x_k| per output; one-hot x bit-exact; fused rows
bit-identical to the separate calls; quantised bytes bit-exact.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import golden_blocks
from tests.gpu_util import assert_rel, dev, empty, host, quantized

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gguf_dequant_matvec_amd as q  # noqa: E402

# (type, M, K): several tiles, ragged tails, every lane-group width, odd Q8_0
# block counts, the smallest legal shapes.
SHAPES = [
    ("q4_k", 1, 256), ("q4_k", 5, 256), ("q4_k", 77, 2048), ("q4_k", 1000, 4096),
    ("q4_k", 300, 14336), ("q4_k", 129, 8192), ("q4_k", 63, 1536),
    ("q6_k", 1, 256), ("q6_k", 50, 256), ("q6_k", 333, 1536), ("q6_k", 1000, 4096),
    ("q6_k", 97, 14336),
    ("q8_0", 1, 32), ("q8_0", 1536, 576), ("q8_0", 37, 224), ("q8_0", 100, 4096),
    ("q8_0", 19, 96),
    # further formats: Q5_K (256-weight super-blocks) and the 32-weight ones
    ("q5_k", 1, 256), ("q5_k", 77, 2048), ("q5_k", 1000, 4096), ("q5_k", 97, 14336),
    ("q4_0", 1, 32), ("q4_0", 300, 4096), ("q4_0", 37, 224),
    ("q4_1", 129, 2048), ("q4_1", 19, 96),
    ("q5_0", 300, 4096), ("q5_0", 37, 224),
    ("q5_1", 129, 2048), ("q5_1", 1, 32),
    ("q8_1", 1536, 576), ("q8_1", 33, 224),
    # 2- and 3-bit K-quants
    ("q2_k", 1, 256), ("q2_k", 77, 2048), ("q2_k", 1000, 4096), ("q2_k", 97, 14336),
    ("q3_k", 1, 256), ("q3_k", 50, 768), ("q3_k", 1000, 4096), ("q3_k", 97, 14336),
    # short rows of 9-32 units take one step of 16 or 32 lanes: the edges of
    # that rule (10, 16, 17, 20 and 32 units; 36 falls back to the fewest-idle group)
    ("q4_k", 300, 1024), ("q4_k", 300, 1280), ("q6_k", 129, 1280), ("q4_k", 77, 2304),
    ("q4_0", 300, 640), ("q5_1", 129, 1024), ("q8_0", 300, 1088),
    # Q4_1 and Q5_1 in two-block units: one 64-lane step (x in registers),
    # several steps, and an odd block count (one-block units)
    ("q4_1", 300, 4096), ("q5_1", 300, 4096), ("q4_1", 97, 14336), ("q5_1", 97, 14336),
    ("q4_1", 50, 4064),
]


def _case(t, M, K, seed):
    b = quantized(t, M, K, seed)
    x = synth.activations(seed + 1, K)
    return b, x


@pytest.mark.parametrize("t,M,K", SHAPES)
def test_dequant_bit_exact(t, M, K):
    b, _ = _case(t, M, K, 100 + M)
    ref = oracle.dequant(t, b, M, K)
    out = empty(M * K)
    q.qmv_dequant(t, dev(b), M, K, out)
    got = host(out).reshape(M, K)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequant_handbuilt_blocks():
    for t, name, blk, expected in golden_blocks.load():
        n = len(expected)
        out = empty(n)
        q.qmv_dequant(t, dev(blk), 1, n, out)
        bad = golden_blocks.matches(host(out), expected)
        assert not bad, (name, bad[:5])


@pytest.mark.parametrize("t,M,K", SHAPES)
def test_qmv_parity(t, M, K):
    b, x = _case(t, M, K, 200 + M)
    y_ref, a_ref = oracle.qmv(t, b, M, K, x)
    y = empty(M)
    q.qmv(t, dev(b), M, K, dev(x), y)
    assert_rel(host(y), y_ref, a_ref, what=f"{t} {M}x{K}")


# Long matrices: from eight rounds of tiles per wave on, a launch numbers its
# workgroups XCD by XCD (a different tile order); every row is checked.
# Shapes cover one and two row slots and lane groups of 4, 8 and 64.
MANY_ROUNDS = [("q8_0", 20000, 4096), ("q4_k", 40000, 4096), ("q4_k", 600000, 256),
               ("q6_k", 140000, 512)]


@pytest.mark.parametrize("t,M,K", MANY_ROUNDS)
def test_qmv_parity_many_rounds(t, M, K):
    b, x = _case(t, M, K, 250)
    y_ref, a_ref = oracle.qmv(t, b, M, K, x)
    y = empty(M)
    q.qmv(t, dev(b), M, K, dev(x), y)
    assert_rel(host(y), y_ref, a_ref, what=f"{t} {M}x{K}")


@pytest.mark.parametrize("t,M,K", [("q4_k", 40, 4096), ("q6_k", 40, 1536), ("q8_0", 40, 576),
                                   ("q8_0", 9, 224), ("q4_k", 33, 14336), ("q5_k", 40, 4096),
                                   ("q4_0", 40, 576), ("q4_1", 40, 576), ("q5_0", 40, 576),
                                   ("q5_1", 40, 576), ("q8_1", 40, 576), ("q2_k", 40, 4096),
                                   ("q3_k", 40, 1536)])
def test_qmv_one_hot_is_exact(t, M, K):
    b, _ = _case(t, M, K, 300)
    W = oracle.dequant(t, b, M, K)
    bd = dev(b)
    for k in sorted({c for c in [0, 1, 17, 31, 32, 63, 64, 127, 128, 200, 255, K - 1] if c < K}):
        x = np.zeros(K, dtype=np.float32)
        x[k] = 1.0
        y = empty(M)
        q.qmv(t, bd, M, K, dev(x), y)
        assert np.array_equal(host(y), W[:, k]), (t, k)


def test_qmv_scaled_integer_x_is_exact():
    """Hand-built integer blocks (d = dmin = 1) and x = 2^-3 * small integers:
    every partial sum is an exactly representable f32, so y is exact."""
    for t, name, blk, expected in golden_blocks.load():
        if not all(v.denominator == 1 for v, _ in expected):
            continue
        n = len(expected)
        x = ((np.arange(n) % 7) - 3).astype(np.float32) * np.float32(0.125)
        y_ref, _ = oracle.qmv(t, blk, 1, n, x)
        y = empty(1)
        q.qmv(t, dev(blk), 1, n, dev(x), y)
        assert float(host(y)[0]) == y_ref[0], name


def test_x_extremes():
    """Large and tiny activations (1e30 .. 1e-30) keep the relative bound."""
    t, M, K = "q4_k", 64, 4096
    b = quantized(t, M, K, 310)
    g = np.random.default_rng(311)
    x = (g.standard_normal(K) * 10.0 ** g.integers(-30, 30, K)).astype(np.float32)
    y_ref, a_ref = oracle.qmv(t, b, M, K, x)
    y = empty(M)
    q.qmv(t, dev(b), M, K, dev(x), y)
    assert_rel(host(y), y_ref, a_ref, what="wide-range x")


@pytest.mark.parametrize("t,segs,K", [
    ("q4_k", (2048, 512, 512), 2048),          # Llama-3.2-1B QKV
    ("q4_k", (8192, 8192), 2048),              # Llama-3.2-1B gate+up
    ("q6_k", (100, 7, 1, 60), 1536),
    ("q8_0", (300, 11, 5), 576),
    ("q4_k", tuple([3] * 8), 4096),            # the most segments
    ("q4_k", (100, 37, 3), 14336),             # long rows, several unit steps
    ("q5_k", (512, 128, 128), 2048),
    ("q4_0", (64, 16, 16), 4096),
    ("q5_1", (33, 7), 224),
    ("q4_1", (300, 77), 4096),                 # two-block units
    ("q5_1", (129, 64, 3), 2048),
    ("q3_k", (512, 128, 128), 2048),
    ("q2_k", (300, 5), 4096),
    # the stack takes two row slots per lane, each segment alone one
    ("q4_k", (4096, 4096), 4096),
    ("q4_k", (600, 300, 129), 1280),           # 20 units: one 32-lane step per row
    ("q8_0", (1000, 536), 576),                # 9 units: one 16-lane step per row
    # long stacks (eight or more rounds of tiles: workgroups numbered XCD by
    # XCD) against segments that stay below that
    ("q4_k", (20000, 13001, 7000), 4096),
    ("q8_0", (9000, 8000, 3001), 4096),
])
def test_fused_rows(t, segs, K):
    M = sum(segs)
    b, x = _case(t, M, K, 400 + len(segs))
    bd, xd = dev(b), dev(x)
    ys = [empty(m) for m in segs]
    q.qmv_fused_rows(t, bd, K, xd, list(segs), ys)
    y_ref, a_ref = oracle.qmv(t, b, M, K, x)
    rb = q.row_bytes(t, K)
    r0 = 0
    for m, ys_ in zip(segs, ys):
        got = host(ys_)
        assert_rel(got, y_ref[r0:r0 + m], a_ref[r0:r0 + m], what=f"segment at {r0}")
        # bit-identical to a separate single-token call on the same rows
        sep = empty(m)
        q.qmv(t, bd[r0 * rb:(r0 + m) * rb], m, K, xd, sep)
        assert np.array_equal(host(sep).view(np.uint32), got.view(np.uint32))
        r0 += m


def _argmax_gpu(t, bd, M, K, xd):
    idx = empty(1, "int32")
    mx = empty(1)
    ws = empty(q.qmv_workspace_bytes(q.OP_ARGMAX, M, K), "uint8")
    q.qmv_argmax(t, bd, M, K, xd, idx, mx, ws)
    return int(host(idx)[0]), float(host(mx)[0])


@pytest.mark.parametrize("t,M,K", [("q6_k", 5000, 4096), ("q4_k", 777, 2048), ("q8_0", 1536, 576),
                                   ("q6_k", 1, 256), ("q6_k", 3001, 1536), ("q4_k", 300, 14336),
                                   ("q8_0", 70, 8192), ("q5_k", 3000, 4096), ("q4_0", 2000, 2048),
                                   ("q8_1", 900, 576), ("q2_k", 2000, 2048), ("q3_k", 1500, 4096)])
def test_argmax(t, M, K):
    b, x = _case(t, M, K, 500 + M)
    y_ref, a_ref = oracle.qmv(t, b, M, K, x)
    i_ref = int(np.argmax(y_ref))
    bd, xd = dev(b), dev(x)
    i, v = _argmax_gpu(t, bd, M, K, xd)
    if M == 1:
        assert i == 0
    elif y_ref[i_ref] - np.sort(y_ref)[-2] > 1e-5 * (a_ref[i_ref] + a_ref[np.argsort(y_ref)[-2]]):
        assert i == i_ref
    else:   # near tie: any member of the near-tie set
        assert y_ref[i_ref] - y_ref[i] <= 1e-5 * (a_ref[i_ref] + a_ref[i])
    assert abs(v - y_ref[i]) <= 1e-5 * a_ref[i]
    # same per-row values as the matvec: argmax of its y, bit for bit
    y = empty(M)
    q.qmv(t, bd, M, K, xd, y)
    yh = host(y)
    assert i == int(np.argmax(yh)) and np.float32(v) == yh[i]


def test_argmax_workspace_reuse_across_grid_sizes():
    """One workspace serves calls of different sizes (so different grids)
    back to back, without a synchronisation between them: every call's result
    matches the argmax of its own matvec."""
    ws = empty(q.qmv_workspace_bytes(q.OP_ARGMAX, 1, 256), "uint8")
    cases = [("q6_k", 3000, 1536), ("q4_k", 5, 256), ("q8_0", 70000, 576), ("q6_k", 1, 256),
             ("q4_k", 777, 2048), ("q6_k", 3000, 1536)]
    outs = []
    for n, (t, M, K) in enumerate(cases):
        b, x = _case(t, M, K, 700 + n)
        bd, xd = dev(b), dev(x)
        idx, mx, y = empty(1, "int32"), empty(1), empty(M)
        q.qmv_argmax(t, bd, M, K, xd, idx, mx, ws)
        q.qmv(t, bd, M, K, xd, y)
        outs.append((idx, mx, y, bd, xd))
    for (t, M, K), (idx, mx, y, _, _) in zip(cases, outs):
        yh = host(y)
        i = int(host(idx)[0])
        assert i == int(np.argmax(yh)) and np.float32(host(mx)[0]) == yh[i], (t, M, K)


def test_argmax_ties_go_low():
    t, M, K = "q6_k", 4000, 1536
    b, x = _case(t, M, K, 600)
    y_ref, _ = oracle.qmv(t, b, M, K, x)
    win = int(np.argmax(y_ref))
    rb = q.row_bytes(t, K)
    b2 = b.copy()
    for r in (win + 1, M - 1, 3):     # exact copies of the winner, one below it
        b2[r * rb:(r + 1) * rb] = b[win * rb:(win + 1) * rb]
    i, _ = _argmax_gpu(t, dev(b2), M, K, dev(x))
    assert i == min(3, win)


@pytest.mark.parametrize("t", ["q8_0", "q4_k", "q6_k"])
def test_quantize_matches_oracle(t):
    M, K = 96, 4096
    w = synth.weights(700, M, K)
    w[3, :256] = 0.0                       # an all-zero block
    w[5, :256] = np.abs(w[5, :256])        # a non-negative block (m = 0)
    ref = oracle.quantize(t, w)
    out = empty(ref.size, "uint8")
    q.qmv_quantize(t, dev(w), M, K, out)
    got = host(out)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, bad[:10]


def test_probe_reads_everything():
    n = 1 << 22
    g = np.random.default_rng(3)
    buf = g.integers(0, 2 ** 32, n // 4, dtype=np.uint32)
    sink = empty(2048, "int32")
    sink.zero_()
    q.qmv_probe_stream_read(dev(buf.view(np.uint8)), n, sink)
    got = np.bitwise_xor.reduce(host(sink).view(np.uint32))
    assert got == np.bitwise_xor.reduce(buf)


def offset_view(a: np.ndarray):
    """A device copy of `a` that starts 4 bytes into its allocation: 4-byte but
    not 16-byte aligned, as a view one f32 into a tensor is."""
    d = torch.empty(a.size + 1, dtype=torch.float32, device="cuda")
    v = d[1:]
    v.copy_(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).ravel()))
    assert v.data_ptr() % 16 != 0 and v.data_ptr() % 4 == 0
    return v


@pytest.mark.parametrize("t,M,K", [("q4_k", 300, 4096), ("q6_k", 97, 1536), ("q8_0", 77, 576),
                                   ("q8_0", 33, 224), ("q4_0", 40, 14336)])
def test_activations_at_four_byte_offset(t, M, K):
    """x needs only 4-byte alignment: the matvec, fused rows and argmax on an
    x that starts one f32 into its buffer equal the aligned results bit for
    bit, and match the oracle."""
    b, x = _case(t, M, K, 700 + M)
    bd = dev(b)
    xa, xo = dev(x), offset_view(x)
    ya, yo = empty(M), empty(M)
    q.qmv(t, bd, M, K, xa, ya)
    q.qmv(t, bd, M, K, xo, yo)
    y_ref, a_ref = oracle.qmv(t, b, M, K, x)
    assert_rel(host(yo), y_ref, a_ref, what=f"{t} {M}x{K} offset x")
    assert np.array_equal(host(ya).view(np.uint32), host(yo).view(np.uint32))
    segs = [M // 2, M - M // 2]
    ys = [empty(m) for m in segs]
    q.qmv_fused_rows(t, bd, K, xo, segs, ys)
    assert np.array_equal(np.concatenate([host(v) for v in ys]).view(np.uint32),
                          host(ya).view(np.uint32))
    idx, mx = empty(1, "int32"), empty(1)
    ws = empty(q.qmv_workspace_bytes(q.OP_ARGMAX, M, K), "uint8")
    q.qmv_argmax(t, bd, M, K, xo, idx, mx, ws)
    yh = host(ya)
    assert int(host(idx)[0]) == int(np.argmax(yh)) and host(mx)[0] == yh.max()


def test_verify_and_prefill_at_four_byte_offset():
    t, M, K = "q4_k", 256, 4096
    b, _ = _case(t, M, K, 720)
    bd = dev(b)
    for n, fn, op in ((8, q.qmv_gemm_n, q.OP_GEMM_N), (40, q.qmv_gemm, q.OP_GEMM)):
        X = synth.activations(721 + n, K, n=n)
        Ya, Yo = empty(n * M), empty(n * M)
        ws = empty(max(q.qmv_workspace_bytes(op, M, K, n), 16), "uint8")
        fn(t, bd, M, K, n, dev(X), Ya, ws)
        fn(t, bd, M, K, n, offset_view(X), Yo, ws)
        assert np.array_equal(host(Ya).view(np.uint32), host(Yo).view(np.uint32)), n
        Yh = host(Yo).reshape(n, M)
        for j in (0, n - 1):
            yr, ar = oracle.qmv(t, b, M, K, X[j])
            assert_rel(Yh[j], yr, ar, what=f"offset X n={n} column {j}")
