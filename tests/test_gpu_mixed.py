"""GPU parity for qmv_fused_rows2: two row stacks of different formats in one
launch (a Q4_K_M QKV: Q and K in Q4_K, V in Q6_K; FlareLLM page, section
"推理层面的深度优化" and BebeLM page, section "量化格式支持").  Every output
must equal, bit for bit, qmv_fused_rows on its own stack, and the oracle
within 1e-5 * sum|w x|."""
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

CASES = [
    ("q4_k", (4096, 1024), "q6_k", (1024,), 4096),      # Llama-8B-shaped Q4_K_M QKV
    ("q6_k", (1024,), "q4_k", (2048, 512), 2048),       # Llama-1B-shaped, V first
    ("q5_k", (37, 3), "q6_k", (5,), 512),               # ragged, tiny
    ("q4_k", (300,), "q5_k", (101, 7), 14336),          # several unit steps per row
]


@pytest.mark.parametrize("t1,s1,t2,s2,K", CASES)
def test_fused_rows2(t1, s1, t2, s2, K):
    b1 = quantized(t1, sum(s1), K, 1200 + K)
    b2 = quantized(t2, sum(s2), K, 1201 + K)
    x = synth.activations(1202 + K, K)
    d1, d2, xd = dev(b1), dev(b2), dev(x)
    y1 = [empty(m) for m in s1]
    y2 = [empty(m) for m in s2]
    q.qmv_fused_rows2(t1, d1, list(s1), y1, t2, d2, list(s2), y2, K, xd)
    for t, b, d, segs, ys in ((t1, b1, d1, s1, y1), (t2, b2, d2, s2, y2)):
        ref = [empty(m) for m in segs]
        q.qmv_fused_rows(t, d, K, xd, list(segs), ref)
        yr, ar = oracle.qmv(t, b, sum(segs), K, x)
        r0 = 0
        for m, got, want in zip(segs, ys, ref):
            g = host(got)
            assert np.array_equal(g.view(np.uint32), host(want).view(np.uint32)), (t, r0)
            assert_rel(g, yr[r0:r0 + m], ar[r0:r0 + m], what=f"{t} segment at {r0}")
            r0 += m
