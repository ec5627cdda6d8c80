"""Pins for the oracle's gated short convolution (BebeLM page, section
"门控短卷积": B, C, x = split(in_proj(h), 3); Bx = B * x; causal depthwise
conv of kernel size 3 with a 2-position state; y = C * conv; out = out_proj(y))
(CPU).

* a token sequence from a zero state: conv_out per channel equals numpy's
  full convolution of the Bx sequence with the reversed taps (a library
  routine), which fixes the causal tap order and the state shift;
* taps (0, 0, 1) reduce y to C * B * x exactly;
* the state after a token is (old newer entry, Bx);
* a hand-built one-hot case with hand-computed numbers;
* out equals numpy's f64 product of the dequantised out_proj with y.
"""
import numpy as np
import pytest

import oracle
import synth


def _setup(t, D, H, seed):
    b = oracle.quantize(t, synth.weights(seed, 3 * D, H))
    w = synth.normal(seed, synth.T_W, (D, 3), 0.5, 7)
    return b, w


@pytest.mark.parametrize("t", ["q4_k", "q8_0"])
def test_sequence_matches_numpy_convolution(t):
    """Tokens 0..T-1 from a zero state, the state carried between tokens as a
    caller would (f32).  At token s, channel c: y = C * conv with conv the
    entry s of numpy's full convolution of the channel's input sequence
    (earlier Bx as stored, i.e. rounded to f32, then the current Bx) with the
    taps reversed -- so tap 2 is the current input and tap 0 the oldest."""
    D, H, T = 48, 256, 6
    b, w = _setup(t, D, H, 51)
    state = np.zeros((D, 2), dtype=np.float32)
    hist = []                                   # stored (f32) Bx of past tokens
    for s in range(T):
        h = synth.activations(60 + s, H)
        r = oracle.short_conv(t, b, D, H, h, w, state)
        yq, _ = oracle.qmv(t, b, 3 * D, H, h)
        assert np.array_equal(r["bx"], yq[:D] * yq[2 * D:])
        for c in range(D):
            seq = np.array([v[c] for v in hist] + [r["bx"][c]], dtype=np.float64)
            conv = np.convolve(seq, w[c, ::-1].astype(np.float64))[s]
            mag = np.convolve(np.abs(seq), np.abs(w[c, ::-1]).astype(np.float64))[s]
            assert abs(r["y"][c] - yq[D + c] * conv) <= 1e-14 * abs(yq[D + c]) * mag + 1e-300
        hist.append(r["bx"].astype(np.float32).astype(np.float64))
        state = r["state"].astype(np.float32)


def test_identity_taps_and_state_shift():
    t, D, H = "q6_k", 32, 256
    b, _ = _setup(t, D, H, 52)
    w = np.tile(np.array([0.0, 0.0, 1.0], dtype=np.float32), (D, 1))
    state = synth.normal(53, synth.T_X, (D, 2), 1.0)
    h = synth.activations(54, H)
    r = oracle.short_conv(t, b, D, H, h, w, state)
    yq, a = oracle.qmv(t, b, 3 * D, H, h)
    assert np.array_equal(r["y"], yq[D:2 * D] * (yq[:D] * yq[2 * D:]))
    assert np.array_equal(r["state"][:, 0], state[:, 1].astype(np.float64))
    assert np.array_equal(r["state"][:, 1], r["bx"])
    assert np.array_equal(r["A"], a)


def test_hand_built_one_hot():
    """D = 1, H = 32, Q8_0 with d = 1: one-hot h at k = 3 selects codes
    B = 3, C = 5, x = -2.  Taps (1/2, 1/4, 2), state (1, -3):
    Bx = -6, conv = 1/2 - 3/4 - 12 = -49/4, y = 5 * -49/4 = -245/4;
    new state (-3, -6)."""
    def row(code):
        codes = [0] * 32
        codes[3] = code
        return bytes([0x00, 0x3C]) + bytes(c & 0xFF for c in codes)
    b = np.frombuffer(row(3) + row(5) + row(-2), dtype=np.uint8)
    h = np.zeros(32, dtype=np.float32)
    h[3] = 1.0
    r = oracle.short_conv("q8_0", b, 1, 32, h, np.array([[0.5, 0.25, 2.0]]), np.array([[1.0, -3.0]]))
    assert r["bx"][0] == -6.0 and r["y"][0] == -245 / 4
    assert list(r["state"][0]) == [-3.0, -6.0]


def test_out_proj_matches_numpy():
    t, D, H = "q4_k", 64, 256
    b, w = _setup(t, D, H, 55)
    ob = oracle.quantize("q4_k", synth.weights(56, H, D)) if D % 256 == 0 else \
        oracle.quantize("q8_0", synth.weights(56, H, D))
    ot = "q4_k" if D % 256 == 0 else "q8_0"
    h = synth.activations(57, H)
    state = synth.normal(58, synth.T_X, (D, 2), 1.0)
    r = oracle.short_conv(t, b, D, H, h, w, state, ot, ob)
    W = oracle.dequant(ot, ob, H, D).astype(np.float64)
    assert np.allclose(r["out"], W @ r["y"], rtol=1e-12, atol=1e-12 * np.abs(W) @ np.abs(r["y"]))
    assert np.allclose(r["a_out"], np.abs(W) @ np.abs(r["y"]), rtol=1e-12)
