"""GPU parity for qmv_short_conv, one token of the gated short convolution
(BebeLM page, section "门控短卷积"): in_proj with both gates, the causal
depthwise convolution and its state shift in one launch, then out_proj.

Bounds, from the matvec's (dB = 1e-5 * sum|w h| of the B row, likewise C, x):
  |dBx|   <= |x| dB + |B| dx + dB dx + 2^-24 |Bx|
  |dconv| <= |w2| |dBx| + 3 * 2^-24 (|w0 s0| + |w1 s1| + |w2 Bx|)
  |dy|    <= |conv| dC + (|C| + dC) |dconv| + 2^-24 |y|
  |dout_i| <= 1e-5 * sum_j |W_ij y_j| + sum_j |W_ij| |dy_j|   (+ rounding)
The new state's first entry is the old second entry bit for bit; the second
is Bx within its bound.  A three-token run carries the GPU's state forward and
checks every token against the oracle fed that same state.
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

U = 2.0 ** -24


class Block:
    def __init__(self, in_t, out_t, D, H, seed):
        self.in_t, self.out_t, self.D, self.H = in_t, out_t, D, H
        self.b_in = quantized(in_t, 3 * D, H, seed)
        self.b_out = quantized(out_t, H, D, seed + 1)
        self.w = synth.normal(seed + 2, synth.T_W, (D, 3), 0.5)
        self.Wout = np.abs(oracle.dequant(out_t, self.b_out, H, D).astype(np.float64))
        self.d_in, self.d_out, self.d_w = dev(self.b_in), dev(self.b_out), dev(self.w)
        self.ws = empty(q.qmv_workspace_bytes(q.OP_SHORT_CONV, D) // 4)

    def step(self, h, state_dev):
        out = empty(self.H)
        q.qmv_short_conv(self.in_t, self.d_in, self.D, self.H, dev(h), self.d_w, state_dev,
                         self.out_t, self.d_out, out, self.ws)
        return host(out), host(self.ws)[:self.D]

    def check(self, h, state):
        D = self.D
        ref = oracle.short_conv(self.in_t, self.b_in, D, self.H, h, self.w, state, self.out_t,
                                self.b_out)
        st = dev(state.astype(np.float32))
        out, y = self.step(h, st)
        new_state = host(st).reshape(D, 2)
        yq, a = oracle.qmv(self.in_t, self.b_in, 3 * D, self.H, h)
        B, C, X = yq[:D], yq[D:2 * D], yq[2 * D:]
        dB, dC, dX = REL * a[:D], REL * a[D:2 * D], REL * a[2 * D:]
        bx = ref["bx"]
        dbx = np.abs(X) * dB + np.abs(B) * dX + dB * dX + U * np.abs(bx)
        w = self.w.astype(np.float64)
        s = state.astype(np.float32).astype(np.float64)
        conv = w[:, 0] * s[:, 0] + w[:, 1] * s[:, 1] + w[:, 2] * bx
        dconv = np.abs(w[:, 2]) * dbx + 3 * U * (np.abs(w[:, 0] * s[:, 0]) + np.abs(w[:, 1] * s[:, 1]) +
                                                 np.abs(w[:, 2] * bx))
        dy = np.abs(conv) * dC + (np.abs(C) + dC) * dconv + U * np.abs(ref["y"]) + 1e-38
        err_y = np.abs(y.astype(np.float64) - ref["y"])
        assert np.all(err_y <= dy), f"y: worst {float(np.max(err_y / dy)):.2f} of the bound"
        assert np.array_equal(new_state[:, 0], state[:, 1].astype(np.float32))
        assert np.all(np.abs(new_state[:, 1] - bx) <= dbx + 1e-38)
        dout = REL * ref["a_out"] + self.Wout @ dy + 4 * U * ref["a_out"] + 1e-38
        err_o = np.abs(out.astype(np.float64) - ref["out"])
        assert np.all(err_o <= dout), f"out: worst {float(np.max(err_o / dout)):.2f} of the bound"
        return new_state


CASES = [
    ("q4_k", "q4_k", 2048, 2048),     # LFM2 shape: in_proj 6144 x 2048, out_proj 2048 x 2048
    ("q8_0", "q8_0", 96, 224),        # ragged tiles, one-block units
    ("q5_k", "q6_k", 256, 512),
    ("q6_k", "q4_0", 160, 1536),
]


@pytest.mark.parametrize("in_t,out_t,D,H", CASES)
def test_short_conv_parity(in_t, out_t, D, H):
    blk = Block(in_t, out_t, D, H, 950 + D)
    state = synth.normal(960 + D, synth.T_X, (D, 2), 1.0).astype(np.float32)
    blk.check(synth.activations(970 + D, H), state)


def test_short_conv_three_tokens_from_zero_state():
    blk = Block("q4_k", "q4_k", 512, 1024, 980)
    state = np.zeros((512, 2), dtype=np.float32)
    for t in range(3):
        state = blk.check(synth.activations(990 + t, 1024), state)
