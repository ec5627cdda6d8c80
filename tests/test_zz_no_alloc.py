"""qmv_argmax_noalloc (the argmax with its keys in a library-owned device
array, for callers that cannot allocate) against qmv_argmax through the C
ABI: two calls in a row, the second on a smaller input, each bit-identical
to qmv_argmax on the same input and matching the oracle's argmax."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev, empty, host, quantized

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gguf_dequant_matvec_amd as q  # noqa: E402


def run_both(t, M, K, seed):
    b = quantized(t, M, K, seed)
    x = synth.activations(seed + 1, K)
    bd, xd = dev(b), dev(x)
    got = []
    for fn in ("ws", "noalloc"):
        idx, mx = empty(1, "int32"), empty(1)
        idx.fill_(-1)
        mx.fill_(float("nan"))
        if fn == "ws":
            ws = empty(q.qmv_workspace_bytes(q.OP_ARGMAX, M, K), "uint8")
            q.qmv_argmax(t, bd, M, K, xd, idx, mx, ws)
        else:
            q.qmv_argmax_noalloc(t, bd, M, K, xd, idx, mx)
        got.append((int(host(idx)[0]), host(mx).view(np.uint32)[0]))
    assert got[0] == got[1], (t, M, K, got)
    y_ref, a_ref = oracle.qmv(t, b, M, K, x)
    order = np.argsort(y_ref)
    top, second = int(order[-1]), int(order[-2])
    if y_ref[top] - y_ref[second] > 1e-5 * (a_ref[top] + a_ref[second]):
        assert got[1][0] == top
    return got[1]


def test_noalloc_two_calls_second_smaller():
    # the first call fills many of the array's keys (a large grid); the
    # second, smaller one must not see any of them
    run_both("q6_k", 60000, 4096, 1201)
    run_both("q6_k", 700, 1536, 1203)


def test_noalloc_formats_and_shapes():
    for t, M, K in (("q4_k", 20000, 4096), ("q8_0", 1536, 576), ("q4_k", 3, 256),
                    ("q5_k", 999, 2048), ("q8_0", 37, 224)):
        run_both(t, M, K, 1210 + M)


def test_noalloc_in_a_graph():
    """Captured in a HIP graph and replayed, with eager calls on other inputs
    between the replays: every replay gives the eager result."""
    t, M, K = "q6_k", 30000, 4096
    b = quantized(t, M, K, 1220)
    bd, xd = dev(b), dev(synth.activations(1221, K))
    idx, mx = empty(1, "int32"), empty(1)
    q.qmv_argmax_noalloc(t, bd, M, K, xd, idx, mx)
    ref = (int(host(idx)[0]), host(mx).view(np.uint32)[0])
    b2 = quantized(t, 5000, K, 1222)
    b2d, x2d = dev(b2), dev(synth.activations(1223, K))
    idx2, mx2 = empty(1, "int32"), empty(1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q.qmv_argmax_noalloc(t, bd, M, K, xd, idx, mx)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.qmv_argmax_noalloc(t, bd, M, K, xd, idx, mx)
    for rep in range(3):
        idx.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert (int(host(idx)[0]), host(mx).view(np.uint32)[0]) == ref, rep
        q.qmv_argmax_noalloc(t, b2d, 5000, K, x2d, idx2, mx2)   # eager work between replays
        torch.cuda.synchronize()
