"""CPU oracle for the dequantize-fused GGUF matvec -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library shares no code with it:
the C source here is compiled with gcc into its own shared object and knows
nothing of HIP.

Every function is a thin numpy wrapper over ``qmv_oracle.c``; see that file
for what each one computes and which passage of the pages it follows.  All
results are float64.

Parity status: every entry point here is pinned by ``tests/test_oracle_*.py``
(hand-built golden blocks, the library float16 codec, round-trip bounds,
exact rational brute force, numpy f64 matmul, scipy's sigmoid, numpy argmax).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

Q4_0 = 2
Q4_1 = 3
Q5_0 = 6
Q5_1 = 7
Q8_0 = 8
Q8_1 = 9
Q2_K = 10
Q3_K = 11
Q4_K = 12
Q5_K = 13
Q6_K = 14
TYPES = {"q4_0": Q4_0, "q4_1": Q4_1, "q5_0": Q5_0, "q5_1": Q5_1, "q8_0": Q8_0, "q8_1": Q8_1,
         "q2_k": Q2_K, "q3_k": Q3_K, "q4_k": Q4_K, "q5_k": Q5_K, "q6_k": Q6_K}

BLOCK_WEIGHTS = {Q4_0: 32, Q4_1: 32, Q5_0: 32, Q5_1: 32, Q8_0: 32, Q8_1: 32,
                 Q2_K: 256, Q3_K: 256, Q4_K: 256, Q5_K: 256, Q6_K: 256}
BLOCK_BYTES = {Q4_0: 18, Q4_1: 20, Q5_0: 22, Q5_1: 24, Q8_0: 34, Q8_1: 36,
               Q2_K: 84, Q3_K: 110, Q4_K: 144, Q5_K: 176, Q6_K: 210}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int32
    ci = ctypes.c_int
    lib.oracle_half_to_float.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_float.restype = ctypes.c_float
    lib.oracle_float_to_half.argtypes = [ctypes.c_float]
    lib.oracle_float_to_half.restype = ctypes.c_uint16
    lib.oracle_dequant.argtypes = [ci, P, i64, i64, P]
    lib.oracle_quantize.argtypes = [ci, P, i64, i64, P]
    lib.oracle_qmv_rows.argtypes = [ci, P, i64, i64, P, i64, P, P, P]
    lib.oracle_qmv.argtypes = [ci, P, i64, i64, P, P, P]
    lib.oracle_argmax.argtypes = [ci, P, i64, i64, P, P, P, P]
    lib.oracle_gate_up_silu.argtypes = [ci, P, i64, i64, P, P, P, P, P, P]
    lib.oracle_short_conv.argtypes = [ci, P, i64, i64, P, P, P, ci, P, P, P, P, P, P, P]
    lib.oracle_gemm_n.argtypes = [ci, P, i64, i64, i32, P, P, P]
    lib.oracle_moe.argtypes = [P, i64, P, P, i32, i32, ci, P, ci, P, i64,
                               P, P, P, P, P, P, P, P, P]
    for name in ("oracle_dequant", "oracle_quantize", "oracle_qmv_rows", "oracle_qmv",
                 "oracle_argmax", "oracle_gate_up_silu", "oracle_short_conv", "oracle_gemm_n",
                 "oracle_moe"):
        getattr(lib, name).restype = ci
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: bad arguments")


def _type(t) -> int:
    return TYPES[t] if isinstance(t, str) else int(t)


def row_bytes(t, K: int) -> int:
    t = _type(t)
    return (K // BLOCK_WEIGHTS[t]) * BLOCK_BYTES[t]


def half_to_float(h: int) -> float:
    return float(_load().oracle_half_to_float(int(h)))


def float_to_half(f: float) -> int:
    return int(_load().oracle_float_to_half(float(f)))


def quantize(t, w: np.ndarray) -> np.ndarray:
    """f32 M x K -> uint8 block buffer (M rows of consecutive blocks)."""
    t = _type(t)
    w = np.ascontiguousarray(w, dtype=np.float32)
    M, K = w.shape
    out = np.zeros(M * row_bytes(t, K), dtype=np.uint8)
    _check(_load().oracle_quantize(t, _ptr(w), M, K, _ptr(out)), "quantize")
    return out


def dequant(t, blocks: np.ndarray, M: int, K: int) -> np.ndarray:
    t = _type(t)
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    assert blocks.size >= M * row_bytes(t, K)
    out = np.empty((M, K), dtype=np.float32)
    _check(_load().oracle_dequant(t, _ptr(blocks), M, K, _ptr(out)), "dequant")
    return out


def qmv(t, blocks: np.ndarray, M: int, K: int, x: np.ndarray):
    """Returns (y, a): f64 row results and f64 sum |w x| per row."""
    t = _type(t)
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.size == K and blocks.size >= M * row_bytes(t, K)
    y = np.empty(M, dtype=np.float64)
    a = np.empty(M, dtype=np.float64)
    _check(_load().oracle_qmv(t, _ptr(blocks), M, K, _ptr(x), _ptr(y), _ptr(a)), "qmv")
    return y, a


def qmv_rows(t, blocks: np.ndarray, M: int, K: int, x: np.ndarray, rows):
    """(y, a) for the listed rows only (sampled checks at full size)."""
    t = _type(t)
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    assert x.size == K and blocks.size >= M * row_bytes(t, K)
    y = np.empty(rows.size, dtype=np.float64)
    a = np.empty(rows.size, dtype=np.float64)
    _check(_load().oracle_qmv_rows(t, _ptr(blocks), M, K, _ptr(x), rows.size, _ptr(rows),
                                   _ptr(y), _ptr(a)), "qmv_rows")
    return y, a


def fused_rows(t, blocks: np.ndarray, K: int, x: np.ndarray, seg_rows):
    """One row stack split into consecutive segments: a list of (y, a) per
    segment, each equal to the plain matvec of its rows (FlareLLM page,
    section "推理层面的深度优化": fused QKV and gate/up projections)."""
    t = _type(t)
    rb = row_bytes(t, K)
    out, r0 = [], 0
    for m in seg_rows:
        out.append(qmv(t, blocks[r0 * rb:(r0 + m) * rb], m, K, x))
        r0 += m
    return out


def gate_up_silu(t, blocks: np.ndarray, I: int, K: int, x: np.ndarray):
    """Gated FFN input from a stacked gate+up matrix of 2I rows (BebeLM page,
    section "核心算子"): returns (h, g, u, a_g, a_u), all f64, with
    h = silu(g) * u and a_g, a_u the rows' sum |w x|."""
    t = _type(t)
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.size == K and blocks.size >= 2 * I * row_bytes(t, K)
    h, g, u, ag, au = (np.empty(I, dtype=np.float64) for _ in range(5))
    _check(_load().oracle_gate_up_silu(t, _ptr(blocks), I, K, _ptr(x), _ptr(h), _ptr(g), _ptr(u),
                                       _ptr(ag), _ptr(au)), "gate_up_silu")
    return h, g, u, ag, au


def short_conv(in_t, in_proj: np.ndarray, D: int, H: int, h: np.ndarray, w_conv: np.ndarray,
               state: np.ndarray, out_t=None, out_proj: np.ndarray = None):
    """One token of the gated short convolution (BebeLM page, section
    "门控短卷积"): returns a dict with y, bx, state (the new one), A (in_proj
    rows' sum |w h|, 3D) and, when out_proj is given, out and a_out; f64."""
    in_t = _type(in_t)
    in_proj = np.ascontiguousarray(in_proj, dtype=np.uint8)
    h = np.ascontiguousarray(h, dtype=np.float32)
    w_conv = np.ascontiguousarray(w_conv, dtype=np.float32).reshape(D, 3)
    state = np.ascontiguousarray(state, dtype=np.float32).reshape(D, 2)
    assert h.size == H and in_proj.size >= 3 * D * row_bytes(in_t, H)
    r = {k: np.empty(n, dtype=np.float64) for k, n in
         (("y", D), ("bx", D), ("state", 2 * D), ("A", 3 * D))}
    out = a_out = None
    ot = 0
    if out_proj is not None:
        ot = _type(out_t)
        out_proj = np.ascontiguousarray(out_proj, dtype=np.uint8)
        assert out_proj.size >= H * row_bytes(ot, D)
        out, a_out = np.empty(H, dtype=np.float64), np.empty(H, dtype=np.float64)
    _check(_load().oracle_short_conv(in_t, _ptr(in_proj), D, H, _ptr(h), _ptr(w_conv), _ptr(state),
                                     ot, _ptr(out_proj), _ptr(r["state"]), _ptr(r["y"]),
                                     _ptr(r["bx"]), _ptr(out), _ptr(a_out), _ptr(r["A"])),
           "short_conv")
    r["state"] = r["state"].reshape(D, 2)
    if out is not None:
        r["out"], r["a_out"] = out, a_out
    return r


def argmax(t, blocks: np.ndarray, M: int, K: int, x: np.ndarray):
    """(index, value, sum|w x| of that row): lowest index among the maxima."""
    t = _type(t)
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    idx = np.zeros(1, dtype=np.int64)
    v = np.zeros(1, dtype=np.float64)
    a = np.zeros(1, dtype=np.float64)
    _check(_load().oracle_argmax(t, _ptr(blocks), M, K, _ptr(x), _ptr(idx), _ptr(v), _ptr(a)),
           "argmax")
    return int(idx[0]), float(v[0]), float(a[0])


def gemm_n(t, blocks: np.ndarray, M: int, K: int, X: np.ndarray):
    """(Y, A) with Y[j, i] = sum_k w_ik X[j, k] in f64, X n x K."""
    t = _type(t)
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    X = np.ascontiguousarray(X, dtype=np.float32)
    n = X.shape[0]
    assert X.shape[1] == K
    Y = np.empty((n, M), dtype=np.float64)
    A = np.empty((n, M), dtype=np.float64)
    _check(_load().oracle_gemm_n(t, _ptr(blocks), M, K, n, _ptr(X), _ptr(Y), _ptr(A)), "gemm_n")
    return Y, A


def moe(x, router, bias, k, gu_t, gate_up, dn_t, down, I):
    """Sigmoid-routed top-k MoE FFN for one token.  Returns a dict with y,
    sel (slot order = descending biased score), w, logits, scores, g, u, h
    (per slot) and a_y (sum over slots of w * sum_j |D[i,j] h_j|)."""
    gu_t, dn_t = _type(gu_t), _type(dn_t)
    x = np.ascontiguousarray(x, dtype=np.float32)
    router = np.ascontiguousarray(router, dtype=np.float32)
    bias = np.ascontiguousarray(bias, dtype=np.float32)
    gate_up = np.ascontiguousarray(gate_up, dtype=np.uint8)
    down = np.ascontiguousarray(down, dtype=np.uint8)
    E, H = router.shape
    assert x.size == H and bias.size == E
    y = np.empty(H, dtype=np.float64)
    sel = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float64)
    logits = np.empty(E, dtype=np.float64)
    scores = np.empty(E, dtype=np.float64)
    g = np.empty((k, I), dtype=np.float64)
    u = np.empty((k, I), dtype=np.float64)
    h = np.empty((k, I), dtype=np.float64)
    a_y = np.empty(H, dtype=np.float64)
    _check(_load().oracle_moe(_ptr(x), H, _ptr(router), _ptr(bias), E, k, gu_t, _ptr(gate_up),
                              dn_t, _ptr(down), I, _ptr(y), _ptr(sel), _ptr(w), _ptr(logits),
                              _ptr(scores), _ptr(g), _ptr(u), _ptr(h), _ptr(a_y)), "moe")
    return dict(y=y, sel=sel, w=w, logits=logits, scores=scores, g=g, u=u, h=h, a_y=a_y)
