// Host-side driver for a sanitizer build of the C ABI layer (qmv_api.cpp):
// every launch function behind the ABI is replaced by a stub that records its
// arguments, so each entry point's host checks, segment tables and dispatch
// run under AddressSanitizer / UndefinedBehaviorSanitizer on the CPU, with no
// GPU and no kernel.  tests/test_oracle_sanitizers.py builds and runs it;
// device pointers here are fake addresses that nothing dereferences.
#include <stdio.h>
#include <string.h>

#include "qmv.h"
#include "qmv_internal.h"
#include "qmv_rows.h"

namespace qmv {
namespace {
int g_calls = 0;
SegTable g_seg{};
int64_t g_M = 0, g_K = 0;
}  // namespace

hipError_t launch_rows_store(int, const uint8_t *, int64_t M, int64_t K, const float *,
                             const SegTable &seg, hipStream_t) {
    g_calls++;
    g_seg = seg;
    g_M = M;
    g_K = K;
    return hipSuccess;
}
hipError_t launch_rows_mixed(int, const uint8_t *, int64_t, const SegTable &, int, const uint8_t *,
                             int64_t, const SegTable &, int64_t, const float *, hipStream_t) {
    g_calls++;
    return hipSuccess;
}
hipError_t launch_rows_silu(int, const uint8_t *, int64_t, int64_t, const float *, float *,
                            hipStream_t) {
    g_calls++;
    return hipSuccess;
}
hipError_t launch_short_conv(int, const uint8_t *, int64_t, int64_t, const float *, const float *,
                             float *, int, const uint8_t *, float *, float *, hipStream_t) {
    g_calls++;
    return hipSuccess;
}
hipError_t launch_rows_argmax(int, const uint8_t *, int64_t, int64_t, const float *, uint64_t *,
                              int32_t *, float *, hipStream_t) {
    g_calls++;
    return hipSuccess;
}
hipError_t launch_rows_argmax_noalloc(int, const uint8_t *, int64_t, int64_t, const float *,
                                      int32_t *, float *, hipStream_t) {
    g_calls++;
    return hipSuccess;
}
hipError_t launch_dequant(int, const uint8_t *, int64_t, int64_t, float *, hipStream_t) {
    g_calls++;
    return hipSuccess;
}
hipError_t launch_quantize(int, const float *, int64_t, int64_t, uint8_t *, hipStream_t) {
    g_calls++;
    return hipSuccess;
}
hipError_t launch_probe(const void *, size_t, uint32_t *, hipStream_t) {
    g_calls++;
    return hipSuccess;
}
hipError_t launch_moe(const float *, int64_t, const float *, const float *, int32_t, int32_t, int,
                      const uint8_t *, int, const uint8_t *, int64_t, float *, int32_t *, float *,
                      uint8_t *, hipStream_t) {
    g_calls++;
    return hipSuccess;
}
hipError_t launch_gemm(int, const uint8_t *, int64_t, int64_t, int64_t, const float *, float *,
                       void *, hipStream_t) {
    g_calls++;
    return hipSuccess;
}
hipError_t launch_gemm_n(int, const uint8_t *, int64_t, int64_t, int32_t, const float *, float *,
                         void *, hipStream_t) {
    g_calls++;
    return hipSuccess;
}
// workspace sizes (the real plans live in the kernel units): fixed sizes,
// enough to exercise the checks; the prefill product always takes one (its
// staged activations), the verify product only when K is split
size_t gemm_workspace(int64_t, int64_t, int64_t) { return 4096; }
size_t gemm_n_workspace(int64_t, int64_t K, int32_t) { return K > 4096 ? 4096 : 0; }
}  // namespace qmv

static int g_fail = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,    \
                    __LINE__, #cond);                                       \
            g_fail++;                                                       \
        }                                                                   \
    } while (0)

int main() {
    using namespace qmv;
    const void *W = (const void *)(uintptr_t)(1 << 20);
    const float *x = (const float *)(uintptr_t)((1 << 20) + 4);  // 4-byte aligned
    float *y = (float *)(uintptr_t)(2 << 20);
    float *ys[QMV_MAX_SEGMENTS + 1];
    int64_t rows[QMV_MAX_SEGMENTS + 1];
    for (int i = 0; i <= QMV_MAX_SEGMENTS; i++) {
        ys[i] = (float *)(uintptr_t)((3 << 20) + 4096 * i);
        rows[i] = 10 + i;
    }
    hipStream_t s = nullptr;

    // single-token calls: every format, good and bad shapes
    const qmv_type types[] = {QMV_Q4_0, QMV_Q4_1, QMV_Q5_0, QMV_Q5_1, QMV_Q8_0, QMV_Q8_1,
                              QMV_Q2_K, QMV_Q3_K, QMV_Q4_K, QMV_Q5_K, QMV_Q6_K};
    qmv_status (*fns[])(const void *, int64_t, int64_t, const float *, float *, hipStream_t) = {
        qmv_q4_0, qmv_q4_1, qmv_q5_0, qmv_q5_1, qmv_q8_0, qmv_q8_1,
        qmv_q2_k, qmv_q3_k, qmv_q4_k, qmv_q5_k, qmv_q6_k};
    for (int i = 0; i < 11; i++) {
        EXPECT(fns[i](W, 7, 256, x, y, s) == QMV_OK);
        EXPECT(fns[i](W, 0, 256, x, y, s) == QMV_ESHAPE);
        EXPECT(fns[i](W, 7, 100, x, y, s) == QMV_ESHAPE);
        EXPECT(fns[i](W, 7, QMV_MAX_K + 256, x, y, s) == QMV_ESHAPE);
        EXPECT(fns[i](nullptr, 7, 256, x, y, s) == QMV_EINVAL);
        EXPECT(fns[i](W, 7, 256, (const float *)((uintptr_t)x + 2), y, s) == QMV_EALIGN);
        EXPECT(qmv_row_bytes(types[i], 256) > 0);
    }
    // fused rows: the segment table reaches the launch as given
    EXPECT(qmv_fused_rows(QMV_Q4_K, W, 4096, x, 3, rows, ys, s) == QMV_OK);
    EXPECT(g_seg.n == 3 && g_seg.start[0] == 0 && g_seg.start[1] == 10 && g_seg.start[3] == 33);
    EXPECT(g_seg.y[2] == ys[2] && g_M == 33 && g_K == 4096);
    EXPECT(qmv_fused_rows(QMV_Q4_K, W, 4096, x, QMV_MAX_SEGMENTS, rows, ys, s) == QMV_OK);
    EXPECT(qmv_fused_rows(QMV_Q4_K, W, 4096, x, QMV_MAX_SEGMENTS + 1, rows, ys, s) == QMV_EINVAL);
    EXPECT(qmv_fused_rows(QMV_Q4_K, W, 4096, x, 0, rows, ys, s) == QMV_EINVAL);
    EXPECT(qmv_fused_rows(QMV_Q4_K, W, 4096, x, 2, nullptr, ys, s) == QMV_EINVAL);
    int64_t bad[2] = {5, 0};
    EXPECT(qmv_fused_rows(QMV_Q4_K, W, 4096, x, 2, bad, ys, s) == QMV_ESHAPE);
    int64_t huge[2] = {0x7FFFFFF0ll, 0x7FFFFFF0ll};
    EXPECT(qmv_fused_rows(QMV_Q4_K, W, 4096, x, 2, huge, ys, s) == QMV_ESHAPE);
    EXPECT(qmv_fused_rows2(QMV_Q4_K, W, 2, rows, ys, QMV_Q6_K, W, 1, rows, ys, 4096, x, s) ==
           QMV_OK);
    EXPECT(qmv_fused_rows2(QMV_Q4_K, W, 2, rows, ys, QMV_Q4_K, W, 1, rows, ys, 4096, x, s) ==
           QMV_EINVAL);
    EXPECT(qmv_gate_up_silu(QMV_Q4_K, W, 64, 4096, x, y, s) == QMV_OK);
    EXPECT(qmv_gate_up_silu(QMV_Q8_0, W, 1 << 20, 32768, x, y, s) == QMV_ESHAPE);

    // workspace-taking calls
    void *ws = (void *)(uintptr_t)(8 << 20);
    const size_t wa = qmv_workspace_bytes(QMV_OP_ARGMAX, 1000, 256, 0, 0);
    EXPECT(qmv_argmax(QMV_Q6_K, W, 1000, 256, x, (int32_t *)y, y + 1, ws, wa, s) == QMV_OK);
    EXPECT(qmv_argmax(QMV_Q6_K, W, 1000, 256, x, (int32_t *)y, y + 1, ws, wa - 1, s) ==
           QMV_EWORKSPACE);
    EXPECT(qmv_argmax_noalloc(QMV_Q6_K, W, 1000, 256, x, (int32_t *)y, y + 1, s) == QMV_OK);
    EXPECT(qmv_argmax_noalloc(QMV_Q6_K, W, 0, 256, x, (int32_t *)y, y + 1, s) == QMV_ESHAPE);
    const size_t wm = qmv_workspace_bytes(QMV_OP_MOE, 2048, 1536, 32, 4);
    EXPECT(moe_qmv_topk(x, 2048, x, x, 32, 4, QMV_Q4_K, W, QMV_Q6_K, W, 1536, y, (int32_t *)y, y,
                        ws, wm, s) == QMV_OK);
    EXPECT(moe_qmv_topk(x, 2048, x, x, 32, 33, QMV_Q4_K, W, QMV_Q6_K, W, 1536, y, (int32_t *)y, y,
                        ws, wm, s) == QMV_ESHAPE);
    const size_t wc = qmv_workspace_bytes(QMV_OP_SHORT_CONV, 2048, 0, 0, 0);
    EXPECT(qmv_short_conv(QMV_Q4_K, W, 2048, 2048, x, x, y, QMV_Q4_K, W, y, ws, wc, s) == QMV_OK);
    EXPECT(qmv_gemm_n(QMV_Q4_K, W, 100, 4096, 8, x, y, nullptr, 0, s) == QMV_OK);
    EXPECT(qmv_gemm_n(QMV_Q4_K, W, 100, 8192, 8, x, y, nullptr, 0, s) == QMV_EWORKSPACE);
    EXPECT(qmv_gemm_n(QMV_Q4_0, W, 100, 4096, 8, x, y, nullptr, 0, s) == QMV_EINVAL);
    EXPECT(qmv_gemm(QMV_Q4_K, W, 100, 4096, 512, x, y, nullptr, 0, s) == QMV_EWORKSPACE);
    EXPECT(qmv_gemm(QMV_Q4_K, W, 100, 4096, 512, x, y, ws, 4096, s) == QMV_OK);
    EXPECT(qmv_gemm(QMV_Q4_K, W, 100, 4096, QMV_MAX_PREFILL_N + 1, x, y, nullptr, 0, s) ==
           QMV_ESHAPE);
    EXPECT(qmv_dequant(QMV_Q4_K, W, 4, 256, (float *)ws, s) == QMV_OK);
    EXPECT(qmv_quantize(QMV_Q5_K, x, 4, 256, (void *)ws, s) == QMV_EINVAL);
    EXPECT(strcmp(qmv_status_str(QMV_EALIGN), "pointer misaligned") == 0);
    if (g_fail) return 1;
    printf("sanitized ABI checks: ok (%d launches reached)\n", g_calls);
    return 0;
}
