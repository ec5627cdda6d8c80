"""Multi-launch entry points inside HIP graphs: the K-split verify and
prefill products (product + ordered reduce), the MoE FFN (router, gate/up,
down) and the stateful short convolution (gates + conv, out_proj).

Each call is captured once, then replayed several times with new inputs
copied into the captured buffers and eager library work between replays.
Every replay must equal, bit for bit, the same call run eagerly on the same
inputs (the library records no memset and keeps no state between calls
besides the caller's convolution state).
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import dev, empty, host, quantized

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gguf_dequant_matvec_amd as q  # noqa: E402


def capture(fn):
    """Warm up on a side stream, then capture fn() in a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def same(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


def replay_check(fn, inputs, outputs, seeds, make_input, noise):
    """For each seed: eager run on new inputs, then a graph replay on the same
    inputs (outputs poisoned first); compare bit for bit."""
    g = capture(fn)
    for rep, seed in enumerate(seeds):
        new = make_input(seed)
        for dst, src in zip(inputs, new):
            dst.copy_(src)
        fn()
        torch.cuda.synchronize()
        ref = [host(o).copy() for o in outputs]
        for o in outputs:
            o.fill_(float("nan")) if o.dtype == torch.float32 else o.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        got = [host(o) for o in outputs]
        for a, b_ in zip(got, ref):
            assert same(a, b_), rep
        noise()                                           # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("kind,t,M,K,n,split", [
    ("verify", "q4_k", 1000, 14336, 16, True),     # 4 K slices + reduce
    ("verify", "q6_k", 500, 8192, 8, True),        # 2 K slices + reduce
    ("verify", "q4_k", 3000, 4096, 8, False),      # one launch
    ("prefill", "q4_k", 256, 14336, 32, True),     # K split (small M, few tokens)
    ("prefill", "q5_k", 129, 4096, 70, True),
])
def test_split_products_replay(kind, t, M, K, n, split):
    b = dev(quantized(t, M, K, 1500 + M))
    X = dev(synth.activations(1501, K, n=n))
    Y = empty(n * M)
    op = q.OP_GEMM_N if kind == "verify" else q.OP_GEMM
    wsb = q.qmv_workspace_bytes(op, M, K, n)
    assert (wsb > 0) == split                            # a K split: two launches
    ws = empty(max(wsb, 16), "uint8")
    other = empty(M)
    x1 = dev(synth.activations(1502, K))

    def fn():
        if kind == "verify":
            q.qmv_gemm_n(t, b, M, K, n, X, Y, ws)
        else:
            q.qmv_gemm(t, b, M, K, n, X, Y, ws)

    replay_check(fn, [X], [Y], [1510, 1511, 1512],
                 lambda s: [dev(synth.activations(s, K, n=n))],
                 lambda: q.qmv(t, b, M, K, x1, other))


def test_moe_replay():
    E, H, I, k = 8, 512, 256, 3
    gu = dev(quantized("q4_k", E * 2 * I, H, 1520))
    dn = dev(quantized("q6_k", E * H, I, 1521))
    R = dev(synth.normal(1522, synth.T_ROUTER, (E, H), 0.05))
    bias = dev(synth.normal(1523, synth.T_BIAS, (E,), synth.BIAS_STD))
    x = dev(synth.activations(1524, H))
    y, idx, w = empty(H), empty(k, "int32"), empty(k)
    ws = empty(q.qmv_workspace_bytes(q.OP_MOE, H, I, E, k), "uint8")
    other = empty(2 * I)

    def fn():
        q.moe_qmv_topk(x, H, R, bias, E, k, "q4_k", gu, "q6_k", dn, I, y, idx, w, ws)

    # different x per replay: the selected experts change between replays
    replay_check(fn, [x], [y, idx, w], [1530, 1531, 1532, 1533],
                 lambda s: [dev(synth.activations(s, H))],
                 lambda: q.qmv("q4_k", gu, 2 * I, H, x, other))


def test_short_conv_replay_carries_state():
    """The convolution state is an input and an output: eager and graph runs
    start from the same state for each token, and both must leave the same
    new state."""
    D, H = 256, 512
    b_in = dev(quantized("q4_k", 3 * D, H, 1540))
    b_out = dev(quantized("q4_k", H, D, 1541))
    wconv = dev(synth.normal(1542, synth.T_W, (D, 3), 0.5))
    h = dev(synth.activations(1543, H))
    state = dev(np.zeros((D, 2), dtype=np.float32))
    out = empty(H)
    ws = empty(q.qmv_workspace_bytes(q.OP_SHORT_CONV, D) // 4)
    other = empty(3 * D)
    g = capture(lambda: q.qmv_short_conv("q4_k", b_in, D, H, h, wconv, state, "q4_k", b_out,
                                         out, ws))
    st = np.zeros((D, 2), dtype=np.float32)
    for rep, seed in enumerate([1550, 1551, 1552]):
        h.copy_(dev(synth.activations(seed, H)))
        state.copy_(dev(st))
        q.qmv_short_conv("q4_k", b_in, D, H, h, wconv, state, "q4_k", b_out, out, ws)
        torch.cuda.synchronize()
        ref_out, ref_state = host(out).copy(), host(state).copy()
        state.copy_(dev(st))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert same(host(out), ref_out), rep
        assert same(host(state), ref_state), rep
        st = ref_state.reshape(D, 2).copy()              # the next token starts here
        q.qmv("q4_k", b_in, 3 * D, H, h, other)          # eager work between replays
        torch.cuda.synchronize()
