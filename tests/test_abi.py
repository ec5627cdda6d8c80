"""CPU checks of the C ABI: libqmv.so loads, exports every function that
include/qmv.h declares, and rejects bad arguments on the host with the
documented status before touching the GPU (no compute call is made)."""
import ctypes
import os
import re

import pytest

import gguf_dequant_matvec_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(q.LIB_PATH), reason="libqmv.so not built")


def declared_functions():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(q.EXPORTS)


def test_every_declared_symbol_is_exported():
    lib = q.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_row_bytes_and_workspace():
    assert q.qmv_row_bytes("q8_0", 576) == 612
    assert q.qmv_row_bytes("q4_k", 4096) == 2304
    assert q.qmv_row_bytes("q6_k", 1536) == 1260
    assert q.qmv_row_bytes("q4_k", 100) == 0
    assert [q.qmv_row_bytes(t, 64) for t in ("q4_0", "q4_1", "q5_0", "q5_1", "q8_1")] == \
        [36, 40, 44, 48, 72]
    assert q.qmv_row_bytes("q5_k", 512) == 352
    assert q.qmv_workspace_bytes(q.OP_ARGMAX, 128000, 4096) >= 8 * 2048
    assert q.qmv_workspace_bytes(q.OP_MOE, 2048, 1536, 32, 4) == 256 + 3 * 4 * 1536 * 4
    # prefill product: whole n x M f32 slices (2 to 16 of them, 256-byte
    # rounded) when K is split, then the staged activations: 1088 bytes per
    # 16 tokens and 256 values (bf16 or f16 hi + lo, sub-block sums) for every
    # token block of 16 * tt tokens (tt = 1, 2 or 4) and 256-weight window
    def staged(n, K, tt):
        return -(-n // (16 * tt)) * -(-K // 256) * 1088 * 16 * tt

    def layouts(M, K, n):
        w = q.qmv_workspace_bytes(q.OP_GEMM, M, K, n)
        out = []
        for tt in (1, 2, 4):
            rest = w - staged(n, K, tt)
            for slices in [0] + list(range(2, 17)):
                if rest == -(-(slices * 4 * n * M) // 256) * 256:
                    out.append((tt, slices))
        return w, out
    # rows and token blocks fill the chip: no split
    for M, K, n in [(28672, 4096, 512), (4096, 4096, 4096), (256, 512, 1)]:
        w, lay = layouts(M, K, n)
        assert any(s == 0 for _, s in lay), (M, K, n, w)
    # few rows and tokens, long K: split
    for M, K, n in [(4096, 14336, 64), (300, 14336, 20)]:
        w, lay = layouts(M, K, n)
        assert any(s >= 2 for _, s in lay), (M, K, n, w)
    w, lay = layouts(4096, 4096, 16)
    assert lay, w
    assert q.qmv_workspace_bytes(q.OP_GEMM, 4096, 4096, q.MAX_PREFILL_N + 1) == 0
    assert q.load().qmv_status_str(3) == b"pointer misaligned"


A16 = 1 << 20      # fake, 16-byte aligned addresses: never dereferenced


def status_of(fn, *args):
    with pytest.raises(q.QmvError) as e:
        fn(*args, stream=0)
    return e.value.status_name


def test_shape_errors():
    assert status_of(q.qmv_q4_k, A16, 0, 256, A16, A16) == "QMV_ESHAPE"
    assert status_of(q.qmv_q4_k, A16, 4, 100, A16, A16) == "QMV_ESHAPE"
    assert status_of(q.qmv_q6_k, A16, 4, 0, A16, A16) == "QMV_ESHAPE"
    assert status_of(q.qmv_q8_0, A16, 4, 48, A16, A16) == "QMV_ESHAPE"
    assert status_of(q.qmv_q8_0, A16, 4, q.MAX_K + 32, A16, A16) == "QMV_ESHAPE"
    assert status_of(q.qmv_q5_k, A16, 4, 128, A16, A16) == "QMV_ESHAPE"
    assert status_of(q.qmv_q2_k, A16, 4, 128, A16, A16) == "QMV_ESHAPE"
    assert status_of(q.qmv_q3_k, A16, 4, 384, A16, A16) == "QMV_ESHAPE"
    assert status_of(q.qmv_q4_0, A16, 4, 48, A16, A16) == "QMV_ESHAPE"
    assert status_of(q.qmv_q5_1, A16, 0, 64, A16, A16) == "QMV_ESHAPE"
    assert status_of(q.qmv_gemm_n, "q4_k", A16, 4, 256, 17, A16, A16, A16, 1 << 20) == "QMV_ESHAPE"
    assert status_of(q.qmv_gemm_n, "q4_k", A16, 4, 256, 0, A16, A16, A16, 1 << 20) == "QMV_ESHAPE"
    assert status_of(q.qmv_fused_rows, "q4_k", A16, 256, A16, [4, 0], [A16, A16]) == "QMV_ESHAPE"
    assert status_of(q.qmv_gate_up_silu, "q4_k", A16, 0, 256, A16, A16) == "QMV_ESHAPE"
    assert status_of(q.qmv_gate_up_silu, "q4_k", A16, 8, 100, A16, A16) == "QMV_ESHAPE"
    # a gate row and its up row must be < 2^31 bytes apart
    assert status_of(q.qmv_gate_up_silu, "q8_0", A16, 1 << 20, 32768, A16, A16) == "QMV_ESHAPE"


def test_pointer_and_type_errors():
    assert status_of(q.qmv_q4_k, 0, 4, 256, A16, A16) == "QMV_EINVAL"
    assert status_of(q.qmv_q4_k, A16, 4, 256, 0, A16) == "QMV_EINVAL"
    assert status_of(q.qmv_dequant, 5, A16, 4, 256, A16) == "QMV_EINVAL"   # no such GGUF type
    assert status_of(q.qmv_dequant, 4, A16, 4, 256, A16) == "QMV_EINVAL"
    assert status_of(q.qmv_dequant, 15, A16, 4, 256, A16) == "QMV_EINVAL"  # Q8_K: not served
    # the matrix-core products take Q8_0, Q4_K, Q5_K and Q6_K, the device
    # quantiser Q8_0, Q4_K and Q6_K
    assert status_of(q.qmv_gemm_n, "q4_0", A16, 4, 256, 8, A16, A16, A16, 1 << 20) == "QMV_EINVAL"
    assert status_of(q.qmv_gemm_n, "q3_k", A16, 4, 256, 8, A16, A16, A16, 1 << 20) == "QMV_EINVAL"
    assert status_of(q.qmv_quantize, "q5_k", A16, 4, 256, A16) == "QMV_EINVAL"
    assert status_of(q.qmv_quantize, "q4_0", A16, 4, 256, A16) == "QMV_EINVAL"
    assert status_of(q.qmv_gemm, "q2_k", A16, 4, 256, 64, A16, A16) == "QMV_EINVAL"
    assert status_of(q.qmv_gemm, "q4_k", A16, 4, 256, 0, A16, A16) == "QMV_ESHAPE"
    assert status_of(q.qmv_gemm, "q4_k", A16, 4, 256, q.MAX_PREFILL_N + 1, A16, A16) == "QMV_ESHAPE"
    assert status_of(q.qmv_gemm, "q4_k", A16, 4, 256, 64, A16 + 2, A16) == "QMV_EALIGN"
    # every plan needs its workspace (the staged activations)
    need = q.qmv_workspace_bytes(q.OP_GEMM, 28672, 4096, 512)
    assert status_of(q.qmv_gemm, "q4_k", A16, 28672, 4096, 512, A16, A16, 0, 0) == "QMV_EWORKSPACE"
    assert status_of(q.qmv_gemm, "q4_k", A16, 28672, 4096, 512, A16, A16, A16,
                     need - 1) == "QMV_EWORKSPACE"
    need = q.qmv_workspace_bytes(q.OP_GEMM, 256, 14336, 32)
    assert need > 0
    assert status_of(q.qmv_gemm, "q4_k", A16, 256, 14336, 32, A16, A16, 0, 0) == "QMV_EWORKSPACE"
    assert status_of(q.qmv_gemm, "q4_k", A16, 256, 14336, 32, A16, A16, A16,
                     need - 1) == "QMV_EWORKSPACE"
    assert status_of(q.qmv_gemm, "q4_k", A16, 256, 14336, 32, A16, A16, A16 + 4,
                     need) == "QMV_EALIGN"
    assert status_of(q.qmv_fused_rows, "q4_k", A16, 256, A16, [1] * 9, [A16] * 9) == "QMV_EINVAL"
    assert status_of(q.qmv_fused_rows, "q4_k", A16, 256, A16, [], []) == "QMV_EINVAL"
    assert status_of(q.qmv_gate_up_silu, "q4_k", A16, 8, 256, A16, 0) == "QMV_EINVAL"
    assert status_of(q.qmv_gate_up_silu, 5, A16, 8, 256, A16, A16) == "QMV_EINVAL"
    # two stacks: distinct formats among Q4_K, Q5_K, Q6_K
    two = ([4], [A16], A16, [4], [A16], 256, A16)
    assert status_of(q.qmv_fused_rows2, "q4_k", A16, *two[:2], "q4_k", *two[2:]) == "QMV_EINVAL"
    assert status_of(q.qmv_fused_rows2, "q8_0", A16, *two[:2], "q6_k", *two[2:]) == "QMV_EINVAL"
    assert status_of(q.qmv_fused_rows2, "q4_k", A16, [0], [A16], "q6_k", A16, [4], [A16], 256,
                     A16) == "QMV_ESHAPE"
    assert status_of(q.qmv_fused_rows2, "q4_k", A16, [4], [A16], "q6_k", A16, [4], [A16], 256,
                     A16 + 2) == "QMV_EALIGN"


def test_alignment_errors():
    # activations (x, X, h, router) and outputs need 4-byte alignment, blocks 2
    assert status_of(q.qmv_q4_k, A16 + 1, 4, 256, A16, A16) == "QMV_EALIGN"
    assert status_of(q.qmv_q4_k, A16, 4, 256, A16 + 2, A16) == "QMV_EALIGN"
    assert status_of(q.qmv_q4_k, A16, 4, 256, A16, A16 + 2) == "QMV_EALIGN"
    assert status_of(q.qmv_gemm_n, "q4_k", A16, 4, 256, 8, A16 + 1, A16, A16, 1 << 20) == \
        "QMV_EALIGN"
    assert status_of(q.qmv_argmax, "q6_k", A16, 4, 256, A16 + 2, A16, A16, A16, 1 << 20) == \
        "QMV_EALIGN"
    assert status_of(q.qmv_gate_up_silu, "q4_k", A16, 8, 256, A16 + 2, A16) == "QMV_EALIGN"
    assert status_of(q.qmv_gate_up_silu, "q4_k", A16, 8, 256, A16, A16 + 2) == "QMV_EALIGN"


def test_workspace_errors():
    ws = q.qmv_workspace_bytes(q.OP_ARGMAX, 1000, 256)
    assert status_of(q.qmv_argmax, "q6_k", A16, 1000, 256, A16, A16, A16, A16, ws - 8) == \
        "QMV_EWORKSPACE"
    assert status_of(q.qmv_argmax, "q6_k", A16, 1000, 256, A16, A16, A16, 0, ws) == \
        "QMV_EWORKSPACE"
    wm = q.qmv_workspace_bytes(q.OP_MOE, 2048, 1536, 32, 4)
    args = (A16, 2048, A16, A16, 32, 4, "q4_k", A16, "q6_k", A16, 1536, A16, A16, A16, A16)
    assert status_of(q.moe_qmv_topk, *args, wm - 4) == "QMV_EWORKSPACE"
    bad_k = (A16, 2048, A16, A16, 32, 33, "q4_k", A16, "q6_k", A16, 1536, A16, A16, A16, A16)
    assert status_of(q.moe_qmv_topk, *bad_k, wm) == "QMV_ESHAPE"
    w64 = q.qmv_workspace_bytes(q.OP_MOE, 256, 64, 4, 2)
    bad_i = (A16, 256, A16, A16, 4, 2, "q8_0", A16, "q8_0", A16, 64, A16, A16, A16, A16)
    assert status_of(q.moe_qmv_topk, *bad_i, w64) == "QMV_ESHAPE"
    wc = q.qmv_workspace_bytes(q.OP_SHORT_CONV, 2048)
    assert wc == 8192
    conv = ("q4_k", A16, 2048, 2048, A16, A16, A16, "q4_k", A16, A16, A16)
    assert status_of(q.qmv_short_conv, *conv, wc - 4) == "QMV_EWORKSPACE"
    assert status_of(q.qmv_short_conv, "q4_k", A16, 0, 2048, A16, A16, A16, "q4_k", A16, A16, A16,
                     wc) == "QMV_ESHAPE"
    # out_proj has D = 100 columns: not a multiple of Q4_K's 256
    assert status_of(q.qmv_short_conv, "q8_0", A16, 100, 256, A16, A16, A16, "q4_k", A16, A16, A16,
                     wc) == "QMV_ESHAPE"
    assert status_of(q.qmv_short_conv, "q4_k", A16, 2048, 2048, A16 + 2, A16, A16, "q4_k", A16, A16,
                     A16, wc) == "QMV_EALIGN"
    assert status_of(q.qmv_short_conv, "q4_k", A16, 2048, 2048, A16, A16, 0, "q4_k", A16, A16, A16,
                     wc) == "QMV_EINVAL"
    # the verify product needs a workspace only when K is split (K > 4096)
    assert q.qmv_workspace_bytes(q.OP_GEMM_N, 4096, 4096, 16) == 0
    assert q.qmv_workspace_bytes(q.OP_GEMM_N, 28672, 4096, 8) == 0
    wg = q.qmv_workspace_bytes(q.OP_GEMM_N, 4096, 14336, 16)
    assert wg == 4 * 16 * 4096 * 4      # four slices of 14 windows
    assert q.qmv_workspace_bytes(q.OP_GEMM_N, 100, q.MAX_K, 5) == 8 * 5 * 100 * 4
    assert status_of(q.qmv_gemm_n, "q4_k", A16, 4096, 14336, 16, A16, A16, A16, wg - 4) == \
        "QMV_EWORKSPACE"


def test_segment_lists_must_match():
    # the binding refuses lists of different lengths before calling the library
    # (it reads nseg entries of both host arrays)
    with pytest.raises(ValueError):
        q.qmv_fused_rows("q4_k", A16, 256, A16, [4, 4], [A16], stream=0)
    with pytest.raises(ValueError):
        q.qmv_fused_rows2("q4_k", A16, [4], [A16, A16], "q6_k", A16, [4], [A16], 256, A16,
                          stream=0)
