"""GPU parity for moe_qmv_topk (sigmoid-routed top-k MoE FFN) against the
oracle, staged so that each stage has its own bound:

 (i)   selection equals the oracle's whenever the oracle's gap between the
       k-th and (k+1)-th biased score is wider than the f32 router can blur
       (2 * 1/4 * 1e-5 * max_e sum|R_e x| + 1e-6; 1/4 is sigmoid's largest
       slope); otherwise the case is ambiguous and only validity is checked;
 (ii)  weights within 1e-6 relative of the oracle's;
 (iii) gate and up rows of each slot within 1e-5 * sum|w x| (the matvec rule);
 (iv)  h = silu(g) * u within 1e-6 relative of silu * up of the GPU's g, u;
 (v)   y within 1e-5 * sum_s w_s sum_j |D_s[i, j] h_j| of the oracle's
       sum_s w_s D_s h_s evaluated on the GPU's own h and w.
BebeLM page, section "核心算子" (MoE FFN).
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

ROUTER_STD = 0.02


class Experts:
    def __init__(self, seed, E, H, I, gu_t, dn_t):
        self.E, self.H, self.I, self.gu_t, self.dn_t = E, H, I, gu_t, dn_t
        self.gu = np.concatenate([quantized(gu_t, 2 * I, H, seed, synth.T_GU, e) for e in range(E)])
        self.dn = np.concatenate([quantized(dn_t, H, I, seed, synth.T_DOWN, e) for e in range(E)])
        self.gu_d, self.dn_d = dev(self.gu), dev(self.dn)
        self.rb_gu = q.row_bytes(gu_t, H)
        self.rb_dn = q.row_bytes(dn_t, I)

    def gu_of(self, e):
        n = 2 * self.I * self.rb_gu
        return self.gu[e * n:(e + 1) * n]

    def dn_of(self, e):
        n = self.H * self.rb_dn
        return self.dn[e * n:(e + 1) * n]


_cache = {}


def experts(key):
    if key not in _cache:
        _cache[key] = Experts(*key)
    return _cache[key]


def run_gpu(ex, x, R, b, k):
    E, H, I = ex.E, ex.H, ex.I
    y = empty(H)
    idx = empty(k, "int32")
    w = empty(k)
    ws = empty(q.qmv_workspace_bytes(q.OP_MOE, H, I, E, k), "uint8")
    q.moe_qmv_topk(dev(x), H, dev(R), dev(b), E, k, ex.gu_t, ex.gu_d, ex.dn_t, ex.dn_d, I,
                   y, idx, w, ws)
    wsh = host(ws)
    logits = wsh[:E * 4].view(np.float32).copy()
    body = wsh[256:].view(np.float32)
    gu = body[:k * 2 * I].reshape(k, 2 * I)
    h = body[k * 2 * I:k * 3 * I].reshape(k, I)
    return dict(y=host(y), idx=host(idx), w=host(w), logits=logits, g=gu[:, :I].copy(),
                u=gu[:, I:].copy(), h=h.copy())


def selection_gap(ref, b, k):
    biased = np.sort(ref["scores"] + b.astype(np.float64))[::-1]
    return biased[k - 1] - biased[k] if k < len(biased) else np.inf


def check_moe(ex, x, R, b, k, strict_selection=True):
    E, H, I = ex.E, ex.H, ex.I
    ref = oracle.moe(x, R, b, k, ex.gu_t, ex.gu, ex.dn_t, ex.dn, I)
    got = run_gpu(ex, x, R, b, k)
    # router logits: the f32 matvec rule against the f64 dot products
    a_r = np.abs(R.astype(np.float64)) @ np.abs(x.astype(np.float64))
    assert_rel(got["logits"], ref["logits"], a_r, what="router logits")
    # (i) selection
    thr = 2 * 0.25 * 1e-5 * a_r.max() + 1e-6
    sel = list(got["idx"])
    assert len(set(sel)) == k and all(0 <= e < E for e in sel)
    if selection_gap(ref, b, k) > thr:
        assert sel == list(ref["sel"]), (sel, list(ref["sel"]))
    elif strict_selection:
        pytest.fail("ambiguous selection for a seed that should be clear")
    # (ii) weights of the GPU's own selection, from the oracle's scores
    s_ref = ref["scores"][sel]
    assert np.allclose(got["w"], s_ref / s_ref.sum(), rtol=1e-6, atol=0)
    assert abs(float(got["w"].astype(np.float64).sum()) - 1.0) <= 1e-6
    # (iii) gate and up rows per slot
    for t, e in enumerate(sel):
        yr, ar = oracle.qmv(ex.gu_t, ex.gu_of(e), 2 * I, H, x)
        assert_rel(got["g"][t], yr[:I], ar[:I], what=f"gate slot {t}")
        assert_rel(got["u"][t], yr[I:], ar[I:], what=f"up slot {t}")
    # (iv) h = silu(g) * u of the GPU's g and u
    g64, u64 = got["g"].astype(np.float64), got["u"].astype(np.float64)
    h_ref = g64 / (1.0 + np.exp(-g64)) * u64
    assert np.all(np.abs(got["h"] - h_ref) <= 1e-6 * np.abs(h_ref) + 1e-30)
    # (v) the weighted down mixture on the GPU's h and w
    y_ref = np.zeros(H)
    a_ref = np.zeros(H)
    for t, e in enumerate(sel):
        yd, ad = oracle.qmv(ex.dn_t, ex.dn_of(e), H, I, got["h"][t])
        y_ref += float(got["w"][t]) * yd
        a_ref += float(got["w"][t]) * ad
    assert_rel(got["y"], y_ref, a_ref, what="down mixture")
    # end to end against the pure oracle, for the record (first-order bound)
    return float(np.max(np.abs(got["y"] - ref["y"]) / np.maximum(ref["a_y"], 1e-30))), ref, got


def lfm2_inputs(seed, E=32, H=2048):
    x = synth.activations(seed, H)
    R = synth.normal(seed, synth.T_ROUTER, (E, H), ROUTER_STD)
    b = synth.normal(seed, synth.T_BIAS, (E,), synth.BIAS_STD)
    return x, R, b


def test_moe_lfm2_shape():
    """The LFM2-style MoE layer: hidden 2048, 32 experts, intermediate 1536,
    top-4, Q4_K gate/up and Q6_K down."""
    ex = experts((3, 32, 2048, 1536, "q4_k", "q6_k"))
    for seed in (3, 33, 333):
        x, R, b = lfm2_inputs(seed)
        e2e, ref, got = check_moe(ex, x, R, b, 4)
        assert e2e < 1e-3


def test_moe_bias_selects_but_does_not_weight():
    ex = experts((3, 32, 2048, 1536, "q4_k", "q6_k"))
    x, R, b = lfm2_inputs(41)
    ref = oracle.moe(x, R, np.zeros(32, np.float32), 4, "q4_k", ex.gu, "q6_k", ex.dn, 1536)
    loser = int(np.argsort(-ref["logits"], kind="stable")[-1])
    b = np.zeros(32, np.float32)
    b[loser] = 5.0
    _, ref2, got = check_moe(ex, x, R, b, 4)
    assert got["idx"][0] == loser
    assert got["w"][0] < 0.25


def test_moe_k1_and_tie_to_lower_expert():
    ex = experts((3, 32, 2048, 1536, "q4_k", "q6_k"))
    x, R, b = lfm2_inputs(42)
    check_moe(ex, x, R, b, 1)
    R2 = R.copy()
    R2[9] = R2[20] = 0.05 * np.sign(x)           # identical, clearly largest rows
    b2 = np.zeros(32, np.float32)
    _, ref, got = check_moe(ex, x, R2, b2, 2)
    assert list(got["idx"]) == [9, 20]
    assert got["w"][0] == got["w"][1]


@pytest.mark.parametrize("E,H,I,k,gu_t,dn_t", [
    (8, 256, 256, 8, "q4_k", "q6_k"),     # k = E: every expert, dense sigmoid mixture
    (8, 512, 256, 3, "q6_k", "q4_k"),
    (5, 256, 128, 2, "q8_0", "q8_0"),     # Q8_0 experts, odd expert count, 1-block units
    (6, 512, 256, 3, "q8_0", "q8_0"),     # Q8_0 experts, 2-block units
    (64, 256, 256, 6, "q4_k", "q8_0"),    # the most experts
    (8, 512, 256, 4, "q5_k", "q4_0"),     # further formats: Q5_K gate/up, Q4_0 down
    (6, 256, 128, 2, "q5_0", "q5_1"),
    (4, 256, 256, 2, "q4_1", "q8_1"),
    (4, 512, 256, 2, "q5_1", "q4_1"),     # Q4_1 down in two-block units (I = 4 units of 64)
    (4, 256, 512, 2, "q4_1", "q5_1"),     # Q5_1 down in two-block units
    (8, 512, 256, 4, "q3_k", "q2_k"),     # 3- and 2-bit K-quants
])
def test_moe_small_shapes(E, H, I, k, gu_t, dn_t):
    ex = experts((50 + E, E, H, I, gu_t, dn_t))
    x = synth.activations(60 + E, H)
    R = synth.normal(60 + E, synth.T_ROUTER, (E, H), ROUTER_STD)
    b = synth.normal(60 + E, synth.T_BIAS, (E,), synth.BIAS_STD)
    check_moe(ex, x, R, b, k, strict_selection=False)


def test_moe_activations_at_four_byte_offset():
    """x and the router need only 4-byte alignment: inputs that start one f32
    into their buffers give the aligned call's outputs bit for bit."""
    ex = experts((3, 32, 2048, 1536, "q4_k", "q6_k"))
    x, R, b = lfm2_inputs(7)
    E, H, I, k = ex.E, ex.H, ex.I, 4

    def off(a):
        d = torch.empty(a.size + 1, dtype=torch.float32, device="cuda")
        d[1:].copy_(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).ravel()))
        assert d[1:].data_ptr() % 16 == 4
        return d[1:]

    outs = []
    for xd, Rd in ((dev(x), dev(R)), (off(x), off(R))):
        y, idx, w = empty(H), empty(k, "int32"), empty(k)
        ws = empty(q.qmv_workspace_bytes(q.OP_MOE, H, I, E, k), "uint8")
        q.moe_qmv_topk(xd, H, Rd, dev(b), E, k, ex.gu_t, ex.gu_d, ex.dn_t, ex.dn_d, I, y, idx, w,
                       ws)
        outs.append((host(y).copy(), host(idx).copy(), host(w).copy()))
    for a, c in zip(*outs):
        assert np.array_equal(np.asarray(a).view(np.uint32), np.asarray(c).view(np.uint32))
