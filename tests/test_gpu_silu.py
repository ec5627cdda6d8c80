"""GPU parity for qmv_gate_up_silu: h[j] = silu(g_j) * u_j over a stacked
gate+up matrix of 2I rows, one launch (BebeLM page, section "核心算子").

Bound: g and u carry the matvec's error (|dg| <= 1e-5 * sum|w x| of the gate
row, likewise u); |silu'| <= 1.1, so
  |dh| <= 1.1 |u| dg + |silu(g)| du + 1.1 dg du + 8 * 2^-24 |h|
where the last term covers the f32 exponential, division and product.
Also: h matches silu(y[j]) * y[I + j] computed on the host in f32 from the
plain matvec of the same stack to a few ulp (g and u are the same bits).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import REL, dev, empty, host, quantized

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gguf_dequant_matvec_amd as q  # noqa: E402


def silu_bound(h_ref, g, u, ag, au):
    dg, du = REL * ag, REL * au
    sg = np.abs(g / (1.0 + np.exp(-g)))
    return 1.1 * np.abs(u) * dg + sg * du + 1.1 * dg * du + 8 * 2.0 ** -24 * np.abs(h_ref) + 1e-38


def check(t, I, K, seed, rows=None):
    b = quantized(t, 2 * I, K, seed)
    x = synth.activations(seed + 1, K)
    bd, xd = dev(b), dev(x)
    h = empty(I)
    q.qmv_gate_up_silu(t, bd, I, K, xd, h)
    hh = host(h).astype(np.float64)
    if rows is None:
        h_ref, g, u, ag, au = oracle.gate_up_silu(t, b, I, K, x)
        sel = np.arange(I)
    else:
        sel = rows
        g, ag = oracle.qmv_rows(t, b, 2 * I, K, x, rows)
        u, au = oracle.qmv_rows(t, b, 2 * I, K, x, rows + I)
        h_ref = g / (1.0 + np.exp(-g)) * u
    err = np.abs(hh[sel] - h_ref)
    bound = silu_bound(h_ref, g, u, ag, au)
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, f"{t} I={I} K={K}: {bad.size} over the bound, first {sel[bad[:5]].tolist()}"
    # same g and u bits as the plain matvec of the stack
    y = empty(2 * I)
    q.qmv(t, bd, 2 * I, K, xd, y)
    yh = host(y)
    g32, u32 = yh[:I], yh[I:]
    h32 = (g32 / (np.float32(1.0) + np.exp(-g32))) * u32
    assert np.all(np.abs(hh - h32.astype(np.float64)) <= 8 * 2.0 ** -24 * np.abs(h32) + 1e-38)
    return float(np.max(err / np.maximum(bound, 1e-300)))


SHAPES = [
    ("q4_k", 300, 4096),   # one unit step per row (activations in registers)
    ("q4_k", 301, 2048),   # two rows per wave, ragged last tile
    ("q4_k", 1, 256),
    ("q6_k", 123, 1536),
    ("q6_k", 64, 4096),
    ("q8_0", 77, 576),
    ("q8_0", 33, 224),     # one 32-weight block per unit
    ("q5_k", 200, 2048),
    ("q4_0", 96, 4096),
    ("q5_1", 45, 224),
    ("q3_k", 150, 2048),
    ("q2_k", 64, 4096),
    ("q4_k", 17000, 4096),  # eight or more rounds of tiles (workgroups numbered XCD by XCD)
]


@pytest.mark.parametrize("t,I,K", SHAPES)
def test_gate_up_silu_parity(t, I, K):
    check(t, I, K, 700 + I)


def test_gate_up_silu_llama8b_sampled():
    I, K = synth.CONFIG4["gate_up"][0], synth.CONFIG4["hidden"]
    g = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, I - 2, I - 1], g.integers(0, I, 256)])).astype(np.int64)
    check("q4_k", I, K, 930, rows)
