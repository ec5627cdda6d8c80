"""Pins for the oracle's gated FFN input h = silu(g) * u over a stacked
gate+up matrix (BebeLM page, section "核心算子") (CPU).

* hand-built Q8_0 blocks (scale 1 or 1/2, chosen codes) with a one-hot x give
  known integer g and u; h must equal g * expit(g) * u with scipy's logistic
  (a library routine), including silu(0) = 0 and negative gates;
* a seeded stack: g and u are rows j and I + j of the oracle's plain matvec
  (the row pairing and the I offset), and h follows from them.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth


def q8_0_row(scale_half_bits: int, codes) -> bytes:
    """One Q8_0 block row of 32 weights: little-endian fp16 scale, 32 int8."""
    assert len(codes) == 32
    return bytes([scale_half_bits & 0xFF, scale_half_bits >> 8]) + bytes(c & 0xFF for c in codes)


@pytest.mark.parametrize("half_bits,scale", [(0x3C00, 1.0), (0x3800, 0.5)])
def test_hand_built_stack_one_hot(half_bits, scale):
    I, K, k = 4, 32, 5
    gate_codes = [-3, 0, 4, 127]
    up_codes = [2, -7, 5, -128]
    rows = []
    for j, c in enumerate(gate_codes + up_codes):
        codes = [((7 * j + 3 * i) % 19) - 9 for i in range(32)]  # filler, never multiplied
        codes[k] = c
        rows.append(q8_0_row(half_bits, codes))
    blocks = np.frombuffer(b"".join(rows), dtype=np.uint8)
    x = np.zeros(K, dtype=np.float32)
    x[k] = 1.0
    h, g, u, ag, au = oracle.gate_up_silu("q8_0", blocks, I, K, x)
    g_exp = np.array(gate_codes, dtype=np.float64) * scale
    u_exp = np.array(up_codes, dtype=np.float64) * scale
    assert np.array_equal(g, g_exp)
    assert np.array_equal(u, u_exp)
    assert np.array_equal(ag, np.abs(g_exp)) and np.array_equal(au, np.abs(u_exp))
    want = g_exp * expit(g_exp) * u_exp
    assert np.allclose(h, want, rtol=1e-15, atol=0.0)
    assert h[1] == 0.0                      # silu(0) = 0
    assert h[0] < 0.0                       # silu(-3 s) < 0, u = 2 s > 0


@pytest.mark.parametrize("t,K", [("q4_k", 512), ("q6_k", 256), ("q8_0", 96)])
def test_pairs_rows_j_and_I_plus_j(t, K):
    I = 37
    b = oracle.quantize(t, synth.weights(41, 2 * I, K))
    x = synth.activations(42, K)
    h, g, u, ag, au = oracle.gate_up_silu(t, b, I, K, x)
    y, a = oracle.qmv(t, b, 2 * I, K, x)
    assert np.array_equal(g, y[:I]) and np.array_equal(u, y[I:])
    assert np.array_equal(ag, a[:I]) and np.array_equal(au, a[I:])
    assert np.allclose(h, y[:I] * expit(y[:I]) * y[I:], rtol=1e-14, atol=0.0)
