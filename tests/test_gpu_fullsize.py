"""Full-size parity: the Llama-8B-shaped decode-step matrices (and the
Llama-3.2-1B-shaped ones) through the same entry points and launch
configuration the benchmark times, checked against the oracle on sampled rows
(first, last, segment edges, and a seeded random sample), the argmax over all
128000 rows, and the n = 16 verify product on sampled rows.  Weights are the
oracle's quantisation of seeded N(0, 0.02) draws, x ~ N(0, 1).

Also: a HIP graph of fused rows + argmax, replayed with eager work in
between, gives the eager results on every replay.
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

C4 = synth.CONFIG4
C2 = synth.CONFIG2


def sample_rows(M, edges=(), n=384, seed=0):
    g = np.random.default_rng(seed)
    rows = set([0, 1, M - 2, M - 1]) | set(int(r) for r in g.integers(0, M, n))
    for e in edges:
        rows |= {e - 1, e, e + 1}
    return np.array(sorted(r for r in rows if 0 <= r < M), dtype=np.int64)


_mats = {}


def mat(t, M, K, seed):
    key = (t, M, K, seed)
    if key not in _mats:
        b = quantized(t, M, K, seed)
        _mats[key] = (b, dev(b))
    return _mats[key]


def check_fused(t, segs, K, seed):
    M = sum(segs)
    b, bd = mat(t, M, K, seed)
    x = synth.activations(seed + 1, K)
    ys = [empty(m) for m in segs]
    q.qmv_fused_rows(t, bd, K, dev(x), list(segs), ys)
    y = np.concatenate([host(v) for v in ys])
    edges = np.cumsum(segs)[:-1]
    rows = sample_rows(M, edges, seed=seed)
    yr, ar = oracle.qmv_rows(t, b, M, K, x, rows)
    return assert_rel(y[rows], yr, ar, what=f"{t} fused {segs}x{K}")


def check_single(t, M, K, seed):
    b, bd = mat(t, M, K, seed)
    x = synth.activations(seed + 1, K)
    y = empty(M)
    q.qmv(t, bd, M, K, dev(x), y)
    rows = sample_rows(M, seed=seed)
    yr, ar = oracle.qmv_rows(t, b, M, K, x, rows)
    return assert_rel(host(y)[rows], yr, ar, what=f"{t} {M}x{K}")


def test_llama8b_qkv_fused():
    check_fused("q4_k", C4["qkv"], C4["hidden"], 900)


def test_llama8b_o():
    check_single("q4_k", C4["o"][0], C4["o"][1], 901)


def test_llama8b_gate_up_fused():
    check_fused("q4_k", C4["gate_up"], C4["hidden"], 902)


def test_llama8b_down():
    check_single("q4_k", C4["down"][0], C4["down"][1], 903)


def test_llama8b_output_argmax_and_logits():
    V, H = C4["vocab"], C4["hidden"]
    b, bd = mat("q6_k", V, H, 904)
    x = synth.activations(905, H)
    y_all, a_all = oracle.qmv("q6_k", b, V, H, x)      # every row, for the argmax
    idx = empty(1, "int32")
    mx = empty(1)
    ws = empty(q.qmv_workspace_bytes(q.OP_ARGMAX, V, H), "uint8")
    xd = dev(x)
    q.qmv_argmax("q6_k", bd, V, H, xd, idx, mx, ws)
    i, v = int(host(idx)[0]), float(host(mx)[0])
    order = np.argsort(y_all)
    top, second = order[-1], order[-2]
    gap = y_all[top] - y_all[second]
    assert gap > 1e-5 * (a_all[top] + a_all[second]), "seed gives a near tie"
    assert i == int(top)
    assert abs(v - y_all[top]) <= 1e-5 * a_all[top]
    y = empty(V)
    q.qmv_q6_k(bd, V, H, xd, y)
    yh = host(y)
    rows = sample_rows(V, seed=906)
    assert_rel(yh[rows], y_all[rows], a_all[rows], what="q6_k output logits")
    assert int(np.argmax(yh)) == i and np.float32(v) == yh[i]


def test_llama8b_verify_n16_gate_up():
    t, M, K, n = "q4_k", sum(C4["gate_up"]), C4["hidden"], 16
    b, bd = mat(t, M, K, 902)
    X = synth.activations(907, K, n=n)
    Y = empty(n * M)
    ws = empty(max(q.qmv_workspace_bytes(q.OP_GEMM_N, M, K, n), 16), "uint8")
    q.qmv_gemm_n(t, bd, M, K, n, dev(X), Y, ws)
    Yh = host(Y).reshape(n, M)
    rows = sample_rows(M, n=96, seed=908)
    for j in range(n):
        yr, ar = oracle.qmv_rows(t, b, M, K, X[j], rows)
        assert_rel(Yh[j, rows], yr, ar, what=f"verify column {j}")


@pytest.mark.parametrize("n", [8, 16])
def test_llama8b_verify_output_projection(n):
    """The Q6_K 128000 x 4096 output projection through the verify product at
    n = 8 and 16 (the largest matrix of the verify pass), on sampled rows."""
    V, H = C4["vocab"], C4["hidden"]
    b, bd = mat("q6_k", V, H, 904)
    X = synth.activations(930 + n, H, n=n)
    Y = empty(n * V)
    ws = empty(max(q.qmv_workspace_bytes(q.OP_GEMM_N, V, H, n), 16), "uint8")
    q.qmv_gemm_n("q6_k", bd, V, H, n, dev(X), Y, ws)
    Yh = host(Y).reshape(n, V)
    rows = sample_rows(V, n=64, seed=940 + n)
    for j in range(n):
        yr, ar = oracle.qmv_rows("q6_k", b, V, H, X[j], rows)
        assert_rel(Yh[j, rows], yr, ar, what=f"q6_k output verify n={n} column {j}")


# The largest K the library accepts: x (and its sub-block sums) fill 129-144
# KB of the 160 KB LDS.  One case per LDS layout of x: Q4_K (64-weight units,
# sums per 32), Q6_K (sums per 16), Q8_0 in two-block and one-block units
# (K = 32768 and 32736, an odd block count) and a 32-weight nibble format.
MAX_K_CASES = [("q4_k", 37, q.MAX_K), ("q6_k", 29, q.MAX_K), ("q8_0", 41, q.MAX_K),
               ("q8_0", 23, q.MAX_K - 32), ("q4_0", 19, q.MAX_K), ("q5_k", 7, q.MAX_K)]


@pytest.mark.parametrize("t,M,K", MAX_K_CASES)
def test_max_k_single_and_argmax(t, M, K):
    b, bd = mat(t, M, K, 950 + M)
    x = synth.activations(951 + M, K)
    y = empty(M)
    xd = dev(x)
    q.qmv(t, bd, M, K, xd, y)
    yr, ar = oracle.qmv(t, b, M, K, x)                    # every row
    assert_rel(host(y), yr, ar, what=f"{t} {M}x{K}")
    idx, mx = empty(1, "int32"), empty(1)
    ws = empty(q.qmv_workspace_bytes(q.OP_ARGMAX, M, K), "uint8")
    q.qmv_argmax(t, bd, M, K, xd, idx, mx, ws)
    yh = host(y)
    i, v = int(host(idx)[0]), host(mx)[0]
    # the argmax of the matvec's own row values, bit for bit
    assert i == int(np.argmax(yh)) and v == yh[i]
    order = np.argsort(yr)
    top, second = int(order[-1]), int(order[-2])
    if yr[top] - yr[second] > 1e-5 * (ar[top] + ar[second]):
        assert i == top


@pytest.mark.parametrize("t,M,n", [("q4_k", 300, 8), ("q6_k", 70, 16), ("q8_0", 50, 5)])
def test_max_k_verify(t, M, n):
    K = q.MAX_K
    b, bd = mat(t, M, K, 960 + M)
    X = synth.activations(961 + M, K, n=n)
    Y = empty(n * M)
    ws = empty(max(q.qmv_workspace_bytes(q.OP_GEMM_N, M, K, n), 16), "uint8")
    q.qmv_gemm_n(t, bd, M, K, n, dev(X), Y, ws)
    Yh = host(Y).reshape(n, M)
    for j in range(n):
        yr, ar = oracle.qmv(t, b, M, K, X[j])
        assert_rel(Yh[j], yr, ar, what=f"{t} verify {M}x{K} column {j}")


@pytest.mark.parametrize("t,M,n", [("q4_k", 300, 40), ("q6_k", 70, 20), ("q8_0", 50, 17),
                                   ("q5_k", 129, 70)])
def test_max_k_prefill(t, M, n):
    """The prefill product at the largest K: its staged activations (128
    windows per token block) and its K slices, checked on every output."""
    K = q.MAX_K
    b, bd = mat(t, M, K, 970 + M)
    X = synth.activations(971 + M, K, n=n)
    Y = empty(n * M)
    ws = empty(q.qmv_workspace_bytes(q.OP_GEMM, M, K, n), "uint8")
    q.qmv_gemm(t, bd, M, K, n, dev(X), Y, ws)
    Yr, Ar = oracle.gemm_n(t, b, M, K, X)
    assert_rel(host(Y), Yr.ravel(), Ar.ravel(), what=f"{t} prefill {M}x{K} n={n}")


def test_max_n_and_k_prefill():
    """The prefill product at the most tokens and the largest K together: X
    is 2^31 bytes, so the 32-bit byte offsets into X (and the staged
    activations of 256 token blocks x 128 windows) run up to their limit.
    X is drawn on the device; sampled tokens (both ends, token-block and
    half-way edges) are checked on every row."""
    t, M, K, n = "q4_k", 40, q.MAX_K, q.MAX_PREFILL_N
    b, bd = mat(t, M, K, 980)
    Xd = synth.normal_device(981, synth.T_X, (n, K), synth.X_STD, "cuda")
    Y = empty(n * M)
    ws = empty(q.qmv_workspace_bytes(q.OP_GEMM, M, K, n), "uint8")
    q.qmv_gemm(t, bd, M, K, n, Xd, Y, ws)
    Yh = host(Y).reshape(n, M)
    for j in [0, 1, 63, 64, 8191, 8192, n - 65, n - 1]:
        xj = host(Xd[j])
        yr, ar = oracle.qmv(t, b, M, K, xj)
        assert_rel(Yh[j], yr, ar, what=f"max n and K, token {j}")
    del Xd, ws


def test_llama1b_decode_matvecs_full():
    H = C2["hidden"]
    check_fused("q4_k", C2["qkv"], H, 910)
    check_fused("q4_k", C2["gate_up"], H, 911)
    t, (M, K) = "q4_k", C2["down"]
    b, bd = mat(t, M, K, 912)
    x = synth.activations(913, K)
    y = empty(M)
    q.qmv(t, bd, M, K, dev(x), y)
    yr, ar = oracle.qmv(t, b, M, K, x)                    # every row
    assert_rel(host(y), yr, ar, what="1b down")


def test_graph_replay_matches_eager():
    """Fused QKV + output argmax captured in a HIP graph and replayed three
    times, with eager library work between replays: every replay equals the
    eager result bit for bit."""
    H = 4096
    segs = [1024, 256, 256]
    bq, bqd = mat("q4_k", sum(segs), H, 920)
    bo, bod = mat("q6_k", 20000, H, 921)
    x = dev(synth.activations(922, H))
    ys = [empty(m) for m in segs]
    idx = empty(1, "int32")
    mx = empty(1)
    ws = empty(q.qmv_workspace_bytes(q.OP_ARGMAX, 20000, H), "uint8")

    def step():
        q.qmv_fused_rows("q4_k", bqd, H, x, segs, ys)
        q.qmv_argmax("q6_k", bod, 20000, H, x, idx, mx, ws)

    step()
    ref = [host(v).copy() for v in ys] + [host(idx).copy(), host(mx).copy()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                            # warm up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = empty(4096)
    for rep in range(3):
        for v in ys:
            v.fill_(float("nan"))
        idx.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        got = [host(v) for v in ys] + [host(idx), host(mx)]
        for a, b_ in zip(got, ref):
            assert np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b_).view(np.uint32)), rep
        q.qmv_q6_k(bod, 4096, H, x, other)               # eager work between replays
        torch.cuda.synchronize()
