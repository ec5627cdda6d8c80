"""Python binding of libqmv.so: dequantize-fused GGUF matvec on MI355X.

Argument marshalling only -- every step runs in the HIP kernels of libqmv.so.
Each function has the name and argument order of the C entry point in
include/qmv.h; tensor arguments may be torch tensors (their data pointer is
passed) or raw integer device addresses.  `stream` defaults to torch's
current stream.  A status other than QMV_OK raises QmvError.

Importing works without a GPU (the library only needs the HIP runtime to be
loadable); the library is never replaced by a CPU fallback: if libqmv.so is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

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

OP_ARGMAX = 1
OP_MOE = 2
OP_GEMM_N = 3
OP_SHORT_CONV = 4
OP_GEMM = 5
MAX_K = 32768
MAX_SEGMENTS = 8
MAX_N = 16
MAX_PREFILL_N = 16384

STATUS = {0: "QMV_OK", 1: "QMV_EINVAL", 2: "QMV_ESHAPE", 3: "QMV_EALIGN",
          4: "QMV_EWORKSPACE", 5: "QMV_EHIP"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmv.so")

# every symbol include/qmv.h declares
EXPORTS = ["qmv_q8_0", "qmv_q4_k", "qmv_q6_k", "qmv_q4_0", "qmv_q4_1", "qmv_q5_0", "qmv_q5_1",
           "qmv_q8_1", "qmv_q5_k", "qmv_q2_k", "qmv_q3_k", "qmv_fused_rows", "qmv_fused_rows2",
           "qmv_gate_up_silu", "qmv_short_conv", "qmv_argmax", "qmv_argmax_noalloc", "moe_qmv_topk", "qmv_gemm_n", "qmv_gemm", "qmv_dequant",
           "qmv_quantize", "qmv_row_bytes", "qmv_workspace_bytes", "qmv_last_hip_error",
           "qmv_status_str", "qmv_probe_stream_read", "qmv_time_next_launch"]


class QmvError(RuntimeError):
    def __init__(self, fn: str, status: int, hip: int = 0):
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        self.hip_error = hip
        msg = f"{fn}: {self.status_name}"
        if status == 5:
            msg += f" (hip error {hip})"
        super().__init__(msg)


_lib = None


def load():
    """Load libqmv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m gguf_dequant_matvec_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32, ci, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int,
                           ctypes.c_size_t)
    sig = {
        "qmv_q8_0": [P, i64, i64, P, P, P],
        "qmv_q4_k": [P, i64, i64, P, P, P],
        "qmv_q6_k": [P, i64, i64, P, P, P],
        "qmv_q4_0": [P, i64, i64, P, P, P],
        "qmv_q4_1": [P, i64, i64, P, P, P],
        "qmv_q5_0": [P, i64, i64, P, P, P],
        "qmv_q5_1": [P, i64, i64, P, P, P],
        "qmv_q8_1": [P, i64, i64, P, P, P],
        "qmv_q5_k": [P, i64, i64, P, P, P],
        "qmv_q2_k": [P, i64, i64, P, P, P],
        "qmv_q3_k": [P, i64, i64, P, P, P],
        "qmv_fused_rows": [ci, P, i64, P, i32, P, P, P],
        "qmv_fused_rows2": [ci, P, i32, P, P, ci, P, i32, P, P, i64, P, P],
        "qmv_gate_up_silu": [ci, P, i64, i64, P, P, P],
        "qmv_short_conv": [ci, P, i64, i64, P, P, P, ci, P, P, P, sz, P],
        "qmv_argmax": [ci, P, i64, i64, P, P, P, P, sz, P],
        "qmv_argmax_noalloc": [ci, P, i64, i64, P, P, P, P],
        "moe_qmv_topk": [P, i64, P, P, i32, i32, ci, P, ci, P, i64, P, P, P, P, sz, P],
        "qmv_gemm_n": [ci, P, i64, i64, i32, P, P, P, sz, P],
        "qmv_gemm": [ci, P, i64, i64, i64, P, P, P, sz, P],
        "qmv_dequant": [ci, P, i64, i64, P, P],
        "qmv_quantize": [ci, P, i64, i64, P, P],
        "qmv_probe_stream_read": [P, sz, P, P],
        "qmv_time_next_launch": [P, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ci
    lib.qmv_row_bytes.argtypes = [ci, i64]
    lib.qmv_row_bytes.restype = sz
    lib.qmv_workspace_bytes.argtypes = [ci, i64, i64, i32, i32]
    lib.qmv_workspace_bytes.restype = sz
    lib.qmv_last_hip_error.argtypes = []
    lib.qmv_last_hip_error.restype = ci
    lib.qmv_status_str.argtypes = [ci]
    lib.qmv_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(a) -> int:
    if a is None:
        return 0
    if isinstance(a, int):
        return a
    return int(a.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return int(torch.cuda.current_stream().cuda_stream)
        return 0
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _type(t) -> int:
    return TYPES[t] if isinstance(t, str) else int(t)


def _call(name: str, *args):
    lib = load()
    st = getattr(lib, name)(*args)
    if st != 0:
        raise QmvError(name, st, lib.qmv_last_hip_error())


def row_bytes(t, K: int) -> int:
    t = _type(t)
    return (K // BLOCK_WEIGHTS[t]) * BLOCK_BYTES[t]


def qmv_row_bytes(t, K: int) -> int:
    return int(load().qmv_row_bytes(_type(t), K))


def qmv_workspace_bytes(op: int, a: int, b: int = 0, c: int = 0, d: int = 0) -> int:
    return int(load().qmv_workspace_bytes(op, a, b, c, d))


def qmv_q8_0(blocks, M, K, x, y, stream=None):
    _call("qmv_q8_0", _ptr(blocks), M, K, _ptr(x), _ptr(y), _stream(stream))


def qmv_q4_k(blocks, M, K, x, y, stream=None):
    _call("qmv_q4_k", _ptr(blocks), M, K, _ptr(x), _ptr(y), _stream(stream))


def qmv_q6_k(blocks, M, K, x, y, stream=None):
    _call("qmv_q6_k", _ptr(blocks), M, K, _ptr(x), _ptr(y), _stream(stream))


def qmv(t, blocks, M, K, x, y, stream=None):
    """Single-token matvec in format t (any of TYPES)."""
    _call("qmv_" + {v: k for k, v in TYPES.items()}[_type(t)], _ptr(blocks), M, K, _ptr(x), _ptr(y),
          _stream(stream))


def qmv_q4_0(blocks, M, K, x, y, stream=None):
    _call("qmv_q4_0", _ptr(blocks), M, K, _ptr(x), _ptr(y), _stream(stream))


def qmv_q4_1(blocks, M, K, x, y, stream=None):
    _call("qmv_q4_1", _ptr(blocks), M, K, _ptr(x), _ptr(y), _stream(stream))


def qmv_q5_0(blocks, M, K, x, y, stream=None):
    _call("qmv_q5_0", _ptr(blocks), M, K, _ptr(x), _ptr(y), _stream(stream))


def qmv_q5_1(blocks, M, K, x, y, stream=None):
    _call("qmv_q5_1", _ptr(blocks), M, K, _ptr(x), _ptr(y), _stream(stream))


def qmv_q8_1(blocks, M, K, x, y, stream=None):
    _call("qmv_q8_1", _ptr(blocks), M, K, _ptr(x), _ptr(y), _stream(stream))


def qmv_q5_k(blocks, M, K, x, y, stream=None):
    _call("qmv_q5_k", _ptr(blocks), M, K, _ptr(x), _ptr(y), _stream(stream))


def qmv_q2_k(blocks, M, K, x, y, stream=None):
    _call("qmv_q2_k", _ptr(blocks), M, K, _ptr(x), _ptr(y), _stream(stream))


def qmv_q3_k(blocks, M, K, x, y, stream=None):
    _call("qmv_q3_k", _ptr(blocks), M, K, _ptr(x), _ptr(y), _stream(stream))


def _check_segments(seg_rows, y_seg):
    # the C entry point reads nseg entries of both host arrays
    if len(seg_rows) != len(y_seg):
        raise ValueError(f"seg_rows has {len(seg_rows)} entries but y_seg has {len(y_seg)}")


def qmv_fused_rows(t, blocks, K, x, seg_rows, y_seg, stream=None):
    _check_segments(seg_rows, y_seg)
    n = len(seg_rows)
    rows = (ctypes.c_int64 * max(n, 1))(*seg_rows)
    ys = (ctypes.c_void_p * max(len(y_seg), 1))(*[_ptr(y) for y in y_seg])
    _call("qmv_fused_rows", _type(t), _ptr(blocks), K, _ptr(x), n,
          ctypes.cast(rows, ctypes.c_void_p), ctypes.cast(ys, ctypes.c_void_p), _stream(stream))


def qmv_fused_rows2(t1, blocks1, seg_rows1, y_seg1, t2, blocks2, seg_rows2, y_seg2, K, x,
                    stream=None):
    def arrays(seg_rows, y_seg):
        _check_segments(seg_rows, y_seg)
        rows = (ctypes.c_int64 * max(len(seg_rows), 1))(*seg_rows)
        ys = (ctypes.c_void_p * max(len(y_seg), 1))(*[_ptr(y) for y in y_seg])
        return rows, ys
    r1, y1 = arrays(seg_rows1, y_seg1)
    r2, y2 = arrays(seg_rows2, y_seg2)
    _call("qmv_fused_rows2", _type(t1), _ptr(blocks1), len(seg_rows1), ctypes.cast(r1, ctypes.c_void_p),
          ctypes.cast(y1, ctypes.c_void_p), _type(t2), _ptr(blocks2), len(seg_rows2),
          ctypes.cast(r2, ctypes.c_void_p), ctypes.cast(y2, ctypes.c_void_p), K, _ptr(x),
          _stream(stream))


def qmv_gate_up_silu(t, blocks, I, K, x, h, stream=None):
    _call("qmv_gate_up_silu", _type(t), _ptr(blocks), I, K, _ptr(x), _ptr(h), _stream(stream))


def qmv_short_conv(in_t, in_proj, D, H, h, w_conv, state, out_t, out_proj, out, workspace,
                   ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _call("qmv_short_conv", _type(in_t), _ptr(in_proj), D, H, _ptr(h), _ptr(w_conv), _ptr(state),
          _type(out_t), _ptr(out_proj), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))


def qmv_argmax(t, blocks, M, K, x, idx_out, max_out, workspace, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _call("qmv_argmax", _type(t), _ptr(blocks), M, K, _ptr(x), _ptr(idx_out), _ptr(max_out),
          _ptr(workspace), ws_bytes, _stream(stream))


def qmv_argmax_noalloc(t, blocks, M, K, x, idx_out, max_out, stream=None):
    _call("qmv_argmax_noalloc", _type(t), _ptr(blocks), M, K, _ptr(x), _ptr(idx_out),
          _ptr(max_out), _stream(stream))


def moe_qmv_topk(x, H, router, bias, E, k, gu_t, gate_up, dn_t, down, I, y, topk_idx, topk_w,
                 workspace, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _call("moe_qmv_topk", _ptr(x), H, _ptr(router), _ptr(bias), E, k, _type(gu_t),
          _ptr(gate_up), _type(dn_t), _ptr(down), I, _ptr(y), _ptr(topk_idx), _ptr(topk_w),
          _ptr(workspace), ws_bytes, _stream(stream))


def qmv_gemm_n(t, blocks, M, K, n, X, Y, workspace=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _call("qmv_gemm_n", _type(t), _ptr(blocks), M, K, n, _ptr(X), _ptr(Y), _ptr(workspace),
          ws_bytes, _stream(stream))


def qmv_gemm(t, blocks, M, K, n, X, Y, workspace=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _call("qmv_gemm", _type(t), _ptr(blocks), M, K, n, _ptr(X), _ptr(Y), _ptr(workspace),
          ws_bytes, _stream(stream))


def qmv_dequant(t, blocks, M, K, w_out, stream=None):
    _call("qmv_dequant", _type(t), _ptr(blocks), M, K, _ptr(w_out), _stream(stream))


def qmv_quantize(t, w, M, K, blocks_out, stream=None):
    _call("qmv_quantize", _type(t), _ptr(w), M, K, _ptr(blocks_out), _stream(stream))


def qmv_probe_stream_read(buf, nbytes, sink, stream=None):
    _call("qmv_probe_stream_read", _ptr(buf), nbytes, _ptr(sink), _stream(stream))


def qmv_time_next_launch(start, stop):
    """Arm the timing hook: the next call's main kernel records its own start
    and end into these events (torch.cuda.Event objects already recorded once,
    or raw hipEvent_t addresses; None disarms)."""
    def h(e):
        if e is None:
            return 0
        return e if isinstance(e, int) else int(e.cuda_event)
    _call("qmv_time_next_launch", h(start), h(stop))
