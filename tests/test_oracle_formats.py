"""Pins for the oracle's block decoders, binary16 codec and quantisers (CPU).

* binary16 decode/encode against numpy's float16 (an independent library codec).
* every decoder against hand-built blocks whose weights were worked out by hand
  (tests/golden/handbuilt_blocks.txt).
* quantise -> dequantise round trips against error bounds computed from the
  f32 inputs alone, code-range checks, and Q8_0 byte idempotence.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import golden_blocks


def test_half_to_float_all_codes():
    codes = np.arange(65536, dtype=np.uint16)
    ref = codes.view(np.float16).astype(np.float32)
    got = np.array([oracle.half_to_float(int(c)) for c in codes], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_float_to_half_matches_numpy():
    g = np.random.default_rng(7)
    vals = [
        g.standard_normal(40000).astype(np.float32) * 0.02,
        g.standard_normal(20000).astype(np.float32) * 1e-6,          # subnormal binary16 range
        g.standard_normal(20000).astype(np.float32) * 3e4,           # near overflow
        (g.integers(0, 1 << 16, 20000) * 2.0 ** -25).astype(np.float32),  # exact ties in subnormals
        (1.0 + (2 * g.integers(0, 1024, 20000) + 1) * 2.0 ** -11).astype(np.float32),  # ties at 1.x
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e30, -1e30, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -14, np.inf, -np.inf], dtype=np.float32),
    ]
    x = np.concatenate(vals)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half(float(v)) for v in x], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


@pytest.mark.parametrize("case", golden_blocks.load(), ids=lambda c: c[1])
def test_handbuilt_blocks(case):
    t, name, blk, expected = case
    w = oracle.dequant(t, blk, 1, len(expected))[0]
    bad = golden_blocks.matches(w, expected)
    assert not bad, [(i, float(w[i]), str(expected[i][0])) for i in bad[:10]]


def test_handbuilt_blocks_in_a_matrix():
    """The decoders index rows of consecutive blocks: a 2 x 512 matrix made of
    four hand-built Q4_K blocks decodes to the four expectations in order."""
    cases = [c for c in golden_blocks.load() if c[0] == "q4_k"]
    a, b = cases[0], cases[1]
    buf = np.concatenate([a[2], b[2], b[2], a[2]])
    w = oracle.dequant("q4_k", buf, 2, 512)
    assert not golden_blocks.matches(w[0, :256], a[3])
    assert not golden_blocks.matches(w[0, 256:], b[3])
    assert not golden_blocks.matches(w[1, :256], b[3])
    assert not golden_blocks.matches(w[1, 256:], a[3])


# ---------------------------------------------------------------------------
# quantiser round trips
# ---------------------------------------------------------------------------

EPS16 = 2.0 ** -11   # binary16 relative rounding


def _blocks_of(w, n):
    return w.reshape(-1, n).astype(np.float64)


def test_q8_0_round_trip_and_idempotence():
    w = synth.weights(11, 64, 4096)
    b = oracle.quantize("q8_0", w)
    wh = oracle.dequant("q8_0", b, 64, 4096)
    wb, whb = _blocks_of(w, 32), _blocks_of(wh, 32)
    d32 = np.abs(wb).max(axis=1, keepdims=True) / 127.0
    bound = d32 * (0.5 + 127 * EPS16) * (1 + 1e-6)
    assert np.all(np.abs(wb - whb) <= bound)
    # byte idempotence: re-quantising the decoded weights gives the same bytes
    b2 = oracle.quantize("q8_0", wh)
    assert np.array_equal(b, b2)


def test_q4_k_round_trip():
    w = synth.weights(12, 64, 4096)
    b = oracle.quantize("q4_k", w)
    wh = oracle.dequant("q4_k", b, 64, 4096)
    wsub, whsub = w.reshape(-1, 8, 32).astype(np.float64), wh.reshape(-1, 8, 32).astype(np.float64)
    lo = np.minimum(0.0, wsub.min(axis=2))                     # per sub-block
    hi = wsub.max(axis=2)
    dmin16 = (-lo).max(axis=1, keepdims=True) / 62.0 * (1 + EPS16)
    s = (hi - lo + dmin16) / 15.0                               # >= the scale the rule picks
    d16 = s.max(axis=1, keepdims=True) / 62.0 * (1 + EPS16)
    step = s + d16                                              # d16 * ceil(s / d16) <= s + d16
    ulp = np.abs(wsub).max(axis=2) * 2.0 ** -23
    bound = (0.5 * step + 4 * ulp)[:, :, None]
    err = np.abs(wsub - whsub)
    assert np.all(err <= bound), float((err - bound).max())
    # the error is a real quantisation error, not zero
    assert err.mean() > 1e-4 * np.abs(wsub).mean()


def test_q6_k_round_trip():
    w = synth.weights(13, 64, 4096)
    b = oracle.quantize("q6_k", w)
    wh = oracle.dequant("q6_k", b, 64, 4096)
    wsub, whsub = w.reshape(-1, 16, 16).astype(np.float64), wh.reshape(-1, 16, 16).astype(np.float64)
    s = np.abs(wsub).max(axis=2) / 31.0
    d16 = s.max(axis=1, keepdims=True) / 126.0 * (1 + EPS16)
    step = s + d16
    ulp = np.abs(wsub).max(axis=2) * 2.0 ** -23
    bound = (0.5 * step + 4 * ulp)[:, :, None]
    err = np.abs(wsub - whsub)
    assert np.all(err <= bound), float((err - bound).max())
    assert err.mean() > 1e-4 * np.abs(wsub).mean()


@pytest.mark.parametrize("t", ["q8_0", "q4_k", "q6_k"])
def test_zero_and_constant_blocks(t):
    K = 256
    z = np.zeros((2, K), dtype=np.float32)
    b = oracle.quantize(t, z)
    if t == "q6_k":
        # q = 0 is stored as 32 (bit 5 set in the high pairs); scales and d are 0
        assert not b.reshape(-1, 210)[:, 192:].any()
    else:
        assert not b.any()                 # all-zero input -> all-zero block bytes
    assert not oracle.dequant(t, b, 2, K).any()
    c = np.full((1, K), 0.0125, dtype=np.float32)
    wh = oracle.dequant(t, oracle.quantize(t, c), 1, K)
    assert np.allclose(wh, 0.0125, rtol=0, atol=0.0125 / 20)


@pytest.mark.parametrize("t", ["q4_k", "q6_k"])
def test_quantiser_uses_every_code_level(t):
    """N(0, 0.02) data spread over the sub-block range reaches the extreme codes
    (0 and 15 for Q4_K, -32 or 31 for Q6_K), so the scales are not loose."""
    w = synth.weights(14, 16, 4096)
    wh = oracle.dequant(t, oracle.quantize(t, w), 16, 4096)
    # decoded values of a sub-block lie on an arithmetic grid; the extreme
    # decoded value of each sub-block sits within one step of the input extreme
    n = 32 if t == "q4_k" else 16
    ws, whs = w.reshape(-1, n), wh.reshape(-1, n)
    span = ws.max(axis=1) - ws.min(axis=1)
    assert np.all(np.abs(whs.max(axis=1) - ws.max(axis=1)) <= span / 8)
    assert np.all(np.abs(whs.min(axis=1) - ws.min(axis=1)) <= span / 8)


# ---------------------------------------------------------------------------
# the 32-weight formats and Q5_K (FlareLLM page, section "量化技术的全面支持";
# BebeLM page, section "局限与未来")
# ---------------------------------------------------------------------------

SYM = {"q4_0": 7, "q5_0": 15, "q8_1": 127}
ASYM = {"q4_1": 15, "q5_1": 31}


@pytest.mark.parametrize("t", sorted(SYM) + sorted(ASYM))
def test_32_weight_round_trip(t):
    """Symmetric rule: d = max|w| / half, codes round(w / d16); the error is
    at most half a step.  Asymmetric rule: m = min w, d = (max - m16) / top;
    the error is half a step plus what the fp16 rounding of m and d can push
    past the clamped ends."""
    w = synth.weights(15, 32, 2048)
    wh = oracle.dequant(t, oracle.quantize(t, w), 32, 2048)
    wb, whb = _blocks_of(w, 32), _blocks_of(wh, 32)
    ulp = np.abs(wb).max(axis=1, keepdims=True) * 2.0 ** -22
    if t in SYM:
        d16 = np.abs(wb).max(axis=1, keepdims=True) / SYM[t] * (1 + EPS16)
        bound = 0.5 * d16 + ulp
    else:
        mn, mx = wb.min(axis=1, keepdims=True), wb.max(axis=1, keepdims=True)
        d16 = (mx - mn) * (1 + 2 * EPS16) / ASYM[t] + np.abs(mn) * EPS16
        bound = 0.5 * d16 + 2 * (np.abs(mn) + (mx - mn)) * EPS16 + ulp
    err = np.abs(wb - whb)
    assert np.all(err <= bound), float((err - bound).max())
    assert err.mean() > 1e-4 * np.abs(wb).mean()


def test_q5_k_round_trip():
    w = synth.weights(16, 64, 4096)
    b = oracle.quantize("q5_k", w)
    wh = oracle.dequant("q5_k", b, 64, 4096)
    wsub, whsub = w.reshape(-1, 8, 32).astype(np.float64), wh.reshape(-1, 8, 32).astype(np.float64)
    lo = np.minimum(0.0, wsub.min(axis=2))
    hi = wsub.max(axis=2)
    dmin16 = (-lo).max(axis=1, keepdims=True) / 62.0 * (1 + EPS16)
    s = (hi - lo + dmin16) / 31.0
    d16 = s.max(axis=1, keepdims=True) / 62.0 * (1 + EPS16)
    step = s + d16
    ulp = np.abs(wsub).max(axis=2) * 2.0 ** -23
    bound = (0.5 * step + 4 * ulp)[:, :, None]
    err = np.abs(wsub - whsub)
    assert np.all(err <= bound), float((err - bound).max())
    # finer than Q4_K on the same data: 31 levels instead of 15
    e4 = np.abs(w - oracle.dequant("q4_k", oracle.quantize("q4_k", w), 64, 4096)).mean()
    assert err.mean() < 0.7 * e4


@pytest.mark.parametrize("t", ["q4_0", "q4_1", "q5_0", "q5_1", "q8_1", "q5_k"])
def test_new_formats_zero_and_constant(t):
    K = 256
    z = np.zeros((2, K), dtype=np.float32)
    assert not oracle.dequant(t, oracle.quantize(t, z), 2, K).any()
    c = np.full((1, K), 0.0125, dtype=np.float32)
    wh = oracle.dequant(t, oracle.quantize(t, c), 1, K)
    assert np.allclose(wh, 0.0125, rtol=0, atol=0.0125 / 20)


@pytest.mark.parametrize("t,lo,hi", [("q4_0", 1, 15), ("q5_0", 1, 31), ("q4_1", 0, 15),
                                     ("q5_1", 0, 31), ("q5_k", 0, 31)])
def test_new_formats_reach_the_extreme_codes(t, lo, hi):
    """On N(0, 0.02) data every block reaches its extreme stored codes: the
    symmetric rule maps +-max|w| to 8 -+ 7 (16 -+ 15), the others min and max
    to 0 and the top code.  Codes are read back from the decoded values."""
    w = synth.weights(17, 8, 1024)
    b = oracle.quantize(t, w)
    wh = oracle.dequant(t, b, 8, 1024).reshape(-1, 32).astype(np.float64)
    ws = w.reshape(-1, 32).astype(np.float64)
    # the extreme decoded values sit within one step of the inputs' extremes
    span = ws.max(axis=1) - ws.min(axis=1)
    assert np.all(np.abs(wh.max(axis=1) - ws.max(axis=1)) <= span / (hi - lo) * 1.01)
    assert np.all(np.abs(wh.min(axis=1) - ws.min(axis=1)) <= span / (hi - lo) * 1.01 +
                  (np.abs(ws).max(axis=1) / (hi // 2) if t in ("q4_0", "q5_0") else 0))


# ---------------------------------------------------------------------------
# Q2_K and Q3_K (FlareLLM page, section "量化技术的全面支持": the K-quant
# series runs from Q2K to Q6K)
# ---------------------------------------------------------------------------

def test_q2_k_round_trip():
    """Per 16-weight sub-block the codes 0..3 span [L, L + 3 step] with
    L = -dmin16*m >= lo - dmin16 and step = d16*sc >= s = (hi - L)/3: every
    weight is within half a step of a level, the step at most s + d16."""
    w = synth.weights(18, 64, 4096)
    wh = oracle.dequant("q2_k", oracle.quantize("q2_k", w), 64, 4096)
    ws = w.reshape(-1, 16, 16).astype(np.float64)
    whs = wh.reshape(-1, 16, 16).astype(np.float64)
    lo = np.minimum(0.0, ws.min(axis=2))
    hi = ws.max(axis=2)
    dmin16 = (-lo).max(axis=1, keepdims=True) / 15.0 * (1 + EPS16)
    s = (hi - lo + dmin16) / 3.0
    d16 = s.max(axis=1, keepdims=True) / 15.0 * (1 + EPS16)
    step = s + d16
    slack = (np.abs(lo).max(axis=1, keepdims=True) + hi) * 4 * EPS16
    bound = (0.5 * step + slack)[:, :, None]
    err = np.abs(ws - whs)
    assert np.all(err <= bound), float((err - bound).max())
    # coarser than Q4_K on the same data (3 levels above the min instead of 15)
    e4 = np.abs(w - oracle.dequant("q4_k", oracle.quantize("q4_k", w), 64, 4096)).mean()
    assert err.mean() > 2.0 * e4


def test_q3_k_round_trip():
    """The weight of largest magnitude in each sub-block lands on code -4 of
    a step d16*sc with |step| >= |v|/4: it is reproduced within half a step
    and every other weight within one step (the far side of -4..3 stops at
    3 steps, |w| <= 4 steps)."""
    w = synth.weights(19, 64, 4096)
    wh = oracle.dequant("q3_k", oracle.quantize("q3_k", w), 64, 4096)
    ws = w.reshape(-1, 16, 16).astype(np.float64)
    whs = wh.reshape(-1, 16, 16).astype(np.float64)
    amax = np.abs(ws).max(axis=2)
    d16 = (amax / 4).max(axis=1, keepdims=True) / 31.0 * (1 + EPS16)
    step = amax / 4 + d16
    err = np.abs(ws - whs)
    assert np.all(err <= (step * (1 + 4 * EPS16))[:, :, None])
    arg = np.abs(ws).argmax(axis=2)
    e_ext = np.take_along_axis(err, arg[:, :, None], axis=2)[:, :, 0]
    assert np.all(e_ext <= 0.5 * step * (1 + 4 * EPS16))
    # the extreme is decoded with its own sign
    v = np.take_along_axis(ws, arg[:, :, None], axis=2)[:, :, 0]
    vh = np.take_along_axis(whs, arg[:, :, None], axis=2)[:, :, 0]
    assert np.all(np.sign(vh) == np.sign(v))
    # between Q2_K and Q4_K on the same data
    e2 = np.abs(w - oracle.dequant("q2_k", oracle.quantize("q2_k", w), 64, 4096)).mean()
    e4 = np.abs(w - oracle.dequant("q4_k", oracle.quantize("q4_k", w), 64, 4096)).mean()
    assert e4 < err.mean() < e2


@pytest.mark.parametrize("t", ["q2_k", "q3_k"])
def test_low_bit_k_zero_and_constant(t):
    K = 512
    z = np.zeros((2, K), dtype=np.float32)
    assert not oracle.dequant(t, oracle.quantize(t, z), 2, K).any()
    c = np.full((1, K), 0.0125, dtype=np.float32)
    wh = oracle.dequant(t, oracle.quantize(t, c), 1, K)
    assert np.allclose(wh, 0.0125, rtol=0, atol=0.0125 / 20)


def test_q3_k_uses_both_scale_signs_and_all_codes():
    """A sub-block whose extreme is positive gets a negative scale, one whose
    extreme is negative a positive scale; the decoded sub-block values then
    take the 8 levels sc*d*(-4..3), read back as integers."""
    w = synth.weights(20, 8, 1024)
    b = oracle.quantize("q3_k", w)
    wh = oracle.dequant("q3_k", b, 8, 1024).reshape(-1, 16).astype(np.float64)
    ws = w.reshape(-1, 16).astype(np.float64)
    v = ws[np.arange(ws.shape[0]), np.abs(ws).argmax(axis=1)]
    assert (v > 0).any() and (v < 0).any()
    seen = set()
    for row, vv in zip(wh, v):
        step = -np.abs(row).max() / 4 * np.sign(vv)   # the extreme decodes to -4*step
        q = row / step
        assert np.allclose(q, np.round(q), atol=1e-6)
        seen.update(np.round(q).astype(int).tolist())
    assert seen == set(range(-4, 4))
