"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and describes workload shapes; it holds none
of the quantised-matvec arithmetic (no block format, no quantiser, no dot
product), so both the oracle side and the GPU side may use it.

Every draw is keyed by (seed, tensor id, layer) through numpy's SeedSequence,
so any tensor can be regenerated on its own.  Weights are N(0, 0.02^2) and
activations N(0, 1), as in the decode workloads the pages describe (BebeLM
page, section "独特的层设计", and the FlareLLM page's benchmark models); the
MoE expert bias is N(0, 0.1^2) so that it changes some selections.
"""
from __future__ import annotations

import numpy as np

W_STD = 0.02
X_STD = 1.0
BIAS_STD = 0.1

# tensor ids
T_W, T_X, T_ROUTER, T_BIAS, T_GU, T_DOWN, T_XN = range(7)


def rng(seed: int, tensor: int, layer: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, layer])))


def normal(seed: int, tensor: int, shape, std: float = 1.0, layer: int = 0) -> np.ndarray:
    """float32 N(0, std^2) of the given shape."""
    g = rng(seed, tensor, layer)
    out = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def weights(seed: int, M: int, K: int, tensor: int = T_W, layer: int = 0) -> np.ndarray:
    return normal(seed, tensor, (M, K), W_STD, layer)


def activations(seed: int, K: int, tensor: int = T_X, layer: int = 0, n: int | None = None):
    shape = (K,) if n is None else (n, K)
    return normal(seed, tensor, shape, X_STD, layer)


def normal_device(seed: int, tensor: int, shape, std: float, device, layer: int = 0):
    """float32 N(0, std^2) drawn on a torch device (bench-sized tensors)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + tensor * 10_007 + layer) & 0x7FFFFFFFFFFFFFFF)
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


# ---------------------------------------------------------------------------
# Workload shapes (rows x columns of each weight matrix, per decode token).
# ---------------------------------------------------------------------------

# Q8_0 single matvec, SmolLM2-135M-sized projection.
CONFIG1 = dict(name="q8_0 1536x576", type="q8_0", M=1536, K=576)

# Llama-3.2-1B-shaped decode matvecs, hidden 2048, all Q4_K.
CONFIG2 = dict(
    name="llama-3.2-1b-shaped decode matvecs (q4_k)",
    hidden=2048,
    qkv=(2048, 512, 512),   # fused Q, K, V rows
    gate_up=(8192, 8192),   # fused gate and up rows
    down=(2048, 8192),      # rows x columns
)

# LFM2-style MoE FFN: hidden 2048, 32 experts, intermediate 1536, top-4.
CONFIG3 = dict(name="lfm2-style moe ffn", H=2048, E=32, I=1536, k=4,
               gu_type="q4_k", dn_type="q6_k")

# Llama-8B-shaped decode step: 32 layers + Q6_K output projection with argmax.
CONFIG4 = dict(
    name="llama-8b-shaped decode step",
    hidden=4096,
    layers=32,
    qkv=(4096, 1024, 1024),
    o=(4096, 4096),
    gate_up=(14336, 14336),
    down=(4096, 14336),
    vocab=128000,
    out_type="q6_k",
)

# Small-batch verify: n columns against the config-4 matrices.
CONFIG5 = dict(name="small-batch verify", n=(8, 16))
