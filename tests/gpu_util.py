"""Helpers for the GPU parity tests: device upload and the 1e-5 sum|w x| rule."""
from __future__ import annotations

import numpy as np

import oracle
import synth

REL = 1e-5   # |y_gpu - y_ref| <= REL * sum_k |w_ik x_k| per output


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.array(a, copy=True, order="C")).cuda()


def empty(n, dtype="float32"):
    import torch
    dt = {"float32": torch.float32, "int32": torch.int32, "uint8": torch.uint8,
          "int64": torch.int64}[dtype]
    return torch.empty(n, dtype=dt, device="cuda")


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def quantized(t, M, K, seed, tensor=synth.T_W, layer=0, chunk_rows=8192):
    """Oracle-quantised N(0, 0.02) weights, generated in row chunks."""
    parts = []
    for r0 in range(0, M, chunk_rows):
        m = min(chunk_rows, M - r0)
        w = synth.normal(seed, tensor, (m, K), synth.W_STD, layer * 1_000_003 + r0)
        parts.append(oracle.quantize(t, w))
    return np.concatenate(parts)


def assert_rel(y_gpu: np.ndarray, y_ref: np.ndarray, a_ref: np.ndarray, rel=REL, what=""):
    y_gpu = y_gpu.astype(np.float64)
    err = np.abs(y_gpu - y_ref)
    bound = rel * a_ref
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, (
        f"{what}: {bad.size} outputs over {rel}*sum|wx|; first {bad[:5].tolist()}, "
        f"worst ratio {float(np.max(err / np.maximum(a_ref, 1e-300))):.3e}")
    zero = a_ref == 0
    assert np.all(y_gpu[zero] == 0.0), f"{what}: nonzero output where sum|wx| = 0"
    return float(np.max(err / np.maximum(a_ref, 1e-300))) if err.size else 0.0
