"""Parser for tests/golden/handbuilt_blocks.txt (hand-built blocks with
hand-computed weights).  Returns (type, name, block bytes, expected values)
with expected values as exact Fractions plus a sign flag for zeros."""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

BLOCK_BYTES = {"q4_0": 18, "q4_1": 20, "q5_0": 22, "q5_1": 24, "q8_0": 34, "q8_1": 36,
               "q2_k": 84, "q3_k": 110, "q4_k": 144, "q5_k": 176, "q6_k": 210}
BLOCK_WEIGHTS = {"q4_0": 32, "q4_1": 32, "q5_0": 32, "q5_1": 32, "q8_0": 32, "q8_1": 32,
                 "q2_k": 256, "q3_k": 256, "q4_k": 256, "q5_k": 256, "q6_k": 256}

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "handbuilt_blocks.txt")


def _value(tok: str):
    if tok == "-0":
        return (Fraction(0), True)
    return (Fraction(tok), False)


def load():
    blocks = []
    cur = None
    with open(PATH, encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] == "block":
                cur = dict(type=parts[1], name=parts[2], bytes=bytearray(BLOCK_BYTES[parts[1]]),
                           default=None, sub={}, w={})
                blocks.append(cur)
            elif parts[0] == "byte":
                cur["bytes"][int(parts[1])] = int(parts[2], 16)
            elif parts[0] == "default":
                cur["default"] = _value(parts[1])
            elif parts[0] == "sub":
                cur["sub"][(int(parts[1]), int(parts[2]))] = _value(parts[3])
            elif parts[0] == "w":
                cur["w"][int(parts[1])] = _value(parts[2])
            else:
                raise ValueError(f"bad fixture line: {line}")
    out = []
    for b in blocks:
        n = BLOCK_WEIGHTS[b["type"]]
        exp = []
        for i in range(n):
            if i in b["w"]:
                exp.append(b["w"][i])
                continue
            v = None
            for (size, j), val in b["sub"].items():
                if size * j <= i < size * (j + 1):
                    v = val
            if v is None:
                v = b["default"]
            assert v is not None, (b["name"], i)
            exp.append(v)
        out.append((b["type"], b["name"], np.frombuffer(bytes(b["bytes"]), dtype=np.uint8), exp))
    return out


def matches(got: np.ndarray, expected) -> list:
    """Indices where the f32 values differ from the exact expectation
    (value, or the sign of a zero)."""
    bad = []
    for i, (val, neg_zero) in enumerate(expected):
        g = float(got[i])
        if Fraction(g) != val:
            bad.append(i)
        elif val == 0 and (np.signbit(np.float32(g)) != neg_zero):
            bad.append(i)
    return bad
