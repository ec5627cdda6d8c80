"""Pins for the oracle's sigmoid-routed top-k MoE FFN (CPU).

BebeLM page, section "核心算子" (MoE FFN): sigmoid router rather than softmax,
top-4 of 32 experts, expert bias used only to select, selected weights
renormalised.  Pinned by:
* one-hot router rows, whose logits are known by hand;
* scipy's expit for the sigmoid and for SiLU;
* numpy's stable argsort for the selection when the bias is zero;
* a bias that flips a choice without changing the weights' formula;
* duplicate router rows (a tie) -> the lower expert index is selected first;
* k = 1 (y is the one expert's output) and k = E with zero bias (the dense
  sigmoid-weighted mixture, computed with numpy matmuls on the dequantised
  experts).
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth

H, I, E = 256, 256, 8


def _experts(seed, E=E, H=H, I=I):
    gu = np.concatenate([oracle.quantize("q4_k", synth.weights(seed, 2 * I, H, synth.T_GU, e))
                         for e in range(E)])
    dn = np.concatenate([oracle.quantize("q6_k", synth.weights(seed, H, I, synth.T_DOWN, e))
                         for e in range(E)])
    return gu, dn


def _dense_expert(gu, dn, e, x):
    rb_gu, rb_dn = oracle.row_bytes("q4_k", H), oracle.row_bytes("q6_k", I)
    G = oracle.dequant("q4_k", gu[e * 2 * I * rb_gu:(e + 1) * 2 * I * rb_gu], 2 * I, H).astype(np.float64)
    D = oracle.dequant("q6_k", dn[e * H * rb_dn:(e + 1) * H * rb_dn], H, I).astype(np.float64)
    gu_out = G @ x.astype(np.float64)
    g, u = gu_out[:I], gu_out[I:]
    h = g * expit(g) * u
    return D @ h, g, u, h, np.abs(D) @ np.abs(h)


@pytest.fixture(scope="module")
def experts():
    return _experts(40)


def test_one_hot_router_logits_and_sigmoid(experts):
    gu, dn = experts
    x = synth.activations(41, H)
    R = np.zeros((E, H), dtype=np.float32)
    cols = [3, 100, 7, 255, 0, 64, 128, 31]
    alpha = np.array([0.5, -1.0, 2.0, 0.25, 1.0, -0.5, 4.0, 1.5], dtype=np.float32)
    for e in range(E):
        R[e, cols[e]] = alpha[e]
    out = oracle.moe(x, R, np.zeros(E, np.float32), 4, "q4_k", gu, "q6_k", dn, I)
    logits = alpha.astype(np.float64) * x[cols].astype(np.float64)
    assert np.array_equal(out["logits"], logits)
    assert np.allclose(out["scores"], expit(logits), rtol=1e-15, atol=0)


def test_selection_without_bias_is_top_logits(experts):
    gu, dn = experts
    x = synth.activations(42, H)
    R = synth.normal(42, synth.T_ROUTER, (E, H), 0.05)
    out = oracle.moe(x, R, np.zeros(E, np.float32), 4, "q4_k", gu, "q6_k", dn, I)
    order = np.argsort(-out["logits"], kind="stable")
    assert list(out["sel"]) == list(order[:4])
    s = out["scores"][out["sel"]]
    assert np.allclose(out["w"], s / s.sum(), rtol=1e-15)
    assert abs(out["w"].sum() - 1.0) <= 4 * 2.0 ** -52


def test_bias_selects_but_does_not_weight(experts):
    gu, dn = experts
    x = synth.activations(43, H)
    R = synth.normal(43, synth.T_ROUTER, (E, H), 0.05)
    base = oracle.moe(x, R, np.zeros(E, np.float32), 4, "q4_k", gu, "q6_k", dn, I)
    loser = int(np.argsort(-base["logits"], kind="stable")[-1])      # lowest score
    bias = np.zeros(E, np.float32)
    bias[loser] = 10.0
    out = oracle.moe(x, R, bias, 4, "q4_k", gu, "q6_k", dn, I)
    assert out["sel"][0] == loser                                    # ranked first by the bias
    s = out["scores"][out["sel"]]
    assert np.allclose(out["w"], s / s.sum(), rtol=1e-15)           # weights from unbiased scores
    assert out["w"][0] < 1.0 / 4                                     # the loser keeps its small weight


def test_tie_goes_to_lower_expert(experts):
    gu, dn = experts
    x = synth.activations(44, H)
    R = synth.normal(44, synth.T_ROUTER, (E, H), 0.05)
    R[6] = R[2] = np.abs(R).max() * np.sign(x)                       # identical, largest rows
    out = oracle.moe(x, R, np.zeros(E, np.float32), 2, "q4_k", gu, "q6_k", dn, I)
    assert list(out["sel"]) == [2, 6]
    assert out["w"][0] == out["w"][1] == 0.5


def test_k1_is_the_expert_output(experts):
    gu, dn = experts
    x = synth.activations(45, H)
    R = synth.normal(45, synth.T_ROUTER, (E, H), 0.05)
    out = oracle.moe(x, R, np.zeros(E, np.float32), 1, "q4_k", gu, "q6_k", dn, I)
    e = int(out["sel"][0])
    assert out["w"][0] == 1.0
    y, g, u, h, ay = _dense_expert(gu, dn, e, x)
    assert np.allclose(out["g"][0], g, rtol=0, atol=1e-12 * np.abs(g).max())
    assert np.allclose(out["u"][0], u, rtol=0, atol=1e-12 * np.abs(u).max())
    assert np.all(np.abs(out["h"][0] - h) <= 1e-12 * np.abs(h).max())
    assert np.all(np.abs(out["y"] - y) <= 1e-11 * ay)


def test_k_equals_e_is_dense_sigmoid_mixture(experts):
    gu, dn = experts
    x = synth.activations(46, H)
    R = synth.normal(46, synth.T_ROUTER, (E, H), 0.05)
    out = oracle.moe(x, R, np.zeros(E, np.float32), E, "q4_k", gu, "q6_k", dn, I)
    s = expit(R.astype(np.float64) @ x.astype(np.float64))
    wts = s / s.sum()
    y = np.zeros(H)
    ay = np.zeros(H)
    for e in range(E):
        ye, _, _, _, ae = _dense_expert(gu, dn, e, x)
        y += wts[e] * ye
        ay += wts[e] * ae
    assert sorted(out["sel"]) == list(range(E))
    assert np.all(np.abs(out["y"] - y) <= 1e-11 * ay)
    assert np.allclose(out["a_y"], ay, rtol=1e-11)
