"""Build libqmv.so in-tree with hipcc for gfx950.

    python -m gguf_dequant_matvec_amd.build [--incremental]

Every .hip/.cpp under csrc/ is compiled to an object in parallel, then linked
into gguf_dequant_matvec_amd/libqmv.so.  The row-kernel launcher
(qmv_rows_inst.hip) is compiled once per (format, mode) pair, so its many
kernels build in parallel units.  Packed-FP32 instructions are turned off
for all device code.  With --incremental an object is rebuilt only when its
source, a header or the flags changed.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libqmv.so")
BUILD_DIR = os.path.join(ROOT, "_build", "qmv")
ARCH = os.environ.get("QMV_OFFLOAD_ARCH", "gfx950")

# row-kernel formats (format structs of qmv_formats.h) and modes (qmv_rows.h)
ROW_FORMATS = ["Q2K", "Q3K", "Q4K", "Q5K", "Q6K", "Q40", "Q41", "Q50", "Q51", "Q81x1",
               "Q80x1", "Q80x2", "Q40x2", "Q50x2", "Q41x2", "Q51x2"]
ROW_MODES = ["kModeStore", "kModeArgmax", "kModeMoeGateUp", "kModeMoeDown", "kModeSiluUp",
             "kModeShortConv"]
INST_SRC = "qmv_rows_inst.hip"


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
              shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libqmv)")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]


def units():
    """(source, object name, extra flags) of every compile."""
    out = []
    for f in sorted(os.listdir(CSRC)):
        if not (f.endswith(".hip") or f.endswith(".cpp")):
            continue
        if f == INST_SRC:
            for mode in ROW_MODES:
                for fmt in ROW_FORMATS:
                    out.append((os.path.join(CSRC, f), f"{f}.{mode}.{fmt}.o",
                                [f"-DQMV_INST_FMT={fmt}", f"-DQMV_INST_MODE={mode}"]))
        else:
            out.append((os.path.join(CSRC, f), f + ".o", []))
    return out


def _headers_digest() -> str:
    h = hashlib.sha256()
    for d in (CSRC, os.path.join(ROOT, "include")):
        for f in sorted(os.listdir(d)):
            if f.endswith(".h"):
                h.update(f.encode())
                with open(os.path.join(d, f), "rb") as fh:
                    h.update(fh.read())
    return h.hexdigest()


def _compile(unit, headers: str, incremental: bool) -> str:
    src, name, extra = unit
    obj = os.path.join(BUILD_DIR, name)
    cmd = [hipcc(), *COMMON, *extra, "-x", "hip", "-c", src, "-o", obj]
    h = hashlib.sha256(headers.encode())
    h.update(" ".join(cmd).encode())
    with open(src, "rb") as fh:
        h.update(fh.read())
    stamp = obj + ".sha"
    key = h.hexdigest()
    if incremental and os.path.exists(obj) and os.path.exists(stamp):
        with open(stamp) as fh:
            if fh.read().strip() == key:
                return obj
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    with open(stamp, "w") as fh:
        fh.write(key)
    return obj


def build(verbose: bool = False, incremental: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    us = units()
    headers = _headers_digest()
    workers = max(1, min(16, os.cpu_count() or 1))
    # the longest compiles first
    us.sort(key=lambda u: (u[0].endswith(INST_SRC), u[1]))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda u: _compile(u, headers, incremental), us))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} ({len(objs)} objects)")
    return OUT


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv[1:])
    sys.exit(0)
