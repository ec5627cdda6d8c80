// C ABI of libqmv: argument checks on the host, then kernel launches on the
// caller's stream.  Nothing here allocates, copies or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <map>
#include <mutex>
#include <utility>

#include "qmv.h"
#include "qmv_internal.h"
#include "qmv_rows.h"

namespace qmv {

namespace {

thread_local int g_last_hip_error = 0;
thread_local TimingHook g_timing_hook;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];
std::mutex g_lds_mutex;
std::map<std::pair<int, const void *>, size_t> g_lds;  // (device, kernel) -> dynamic LDS limit set
std::mutex g_occ_mutex;
std::map<std::pair<const void *, size_t>, int> g_occ;  // (kernel, lds) -> blocks per CU

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_type(int t) { return block_weights_of(t) != 0; }
// formats with a verify-product kernel and a device quantiser
bool core_type(int t) { return t == kQ80 || t == kQ4K || t == kQ6K; }
// formats of the matrix-core products (verify and prefill)
bool mfma_type(int t) { return core_type(t) || t == kQ5K; }

qmv_status check_matrix(int t, const void *blocks, int64_t M, int64_t K) {
    if (!valid_type(t)) return QMV_EINVAL;
    if (!blocks) return QMV_EINVAL;
    if (M < 1 || K < 1 || K > QMV_MAX_K || K % block_weights_of(t) != 0) return QMV_ESHAPE;
    if (M > 0x7FFFFFFFll) return QMV_ESHAPE;
    if (!aligned(blocks, 2)) return QMV_EALIGN;
    return QMV_OK;
}

qmv_status from_hip(hipError_t e) {
    if (e == hipSuccess) return QMV_OK;
    g_last_hip_error = (int)e;
    return QMV_EHIP;
}

}  // namespace

void set_timing_hook(hipEvent_t start, hipEvent_t stop) {
    g_timing_hook.start = start;
    g_timing_hook.stop = stop;
}

TimingHook take_timing_hook() {
    TimingHook h = g_timing_hook;
    g_timing_hook = TimingHook{};
    return h;
}

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
        v = 256;
    g_cu_count[dev].store(v, std::memory_order_relaxed);
    return v;
}

int resident_blocks(const void *kernel, int threads, size_t lds) {
    std::lock_guard<std::mutex> lock(g_occ_mutex);
    auto key = std::make_pair(kernel, lds);
    auto it = g_occ.find(key);
    if (it != g_occ.end()) return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds) != hipSuccess) {
        (void)hipGetLastError();  // handled here: do not report it with the next launch
        n = 1;
    }
    if (n < 1) n = 1;
    g_occ[key] = n;
    return n;
}

hipError_t ensure_lds(const void *kernel, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_lds_mutex);
    size_t &done = g_lds[std::make_pair(dev, kernel)];
    if (done >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) done = bytes;
    return e;
}

}  // namespace qmv

using namespace qmv;

extern "C" {

size_t qmv_row_bytes(qmv_type t, int64_t K) {
    if (!valid_type(t) || K < 1 || K % block_weights_of(t) != 0) return 0;
    return row_bytes_of(t, K);
}

size_t qmv_workspace_bytes(qmv_op op, int64_t a, int64_t b, int32_t c, int32_t d) {
    (void)a;
    (void)b;
    if (op == QMV_OP_ARGMAX) return (size_t)kMaxGrid * sizeof(uint64_t);
    if (op == QMV_OP_MOE) {
        if (b < 1 || c < 1 || d < 1) return 0;
        // logits[E] padded to 256 B, then gu[k][2I] and h[k][I] in f32
        return 256 + 3 * (size_t)d * (size_t)b * sizeof(float);
    }
    if (op == QMV_OP_SHORT_CONV) {
        if (a < 1) return 0;
        return ((size_t)a * sizeof(float) + 15) / 16 * 16;  // y[D]
    }
    if (op == QMV_OP_GEMM_N) {
        if (a < 1 || b < 1 || c < 1 || c > QMV_MAX_N) return 0;
        return gemm_n_workspace(a, b, c);
    }
    if (op == QMV_OP_GEMM) {
        if (a < 1 || b < 1 || c < 1 || c > QMV_MAX_PREFILL_N) return 0;
        return gemm_workspace(a, b, c);
    }
    return 0;
}

int qmv_last_hip_error(void) { return g_last_hip_error; }

const char *qmv_status_str(qmv_status s) {
    switch (s) {
    case QMV_OK: return "ok";
    case QMV_EINVAL: return "invalid argument";
    case QMV_ESHAPE: return "shape out of range";
    case QMV_EALIGN: return "pointer misaligned";
    case QMV_EWORKSPACE: return "workspace too small";
    case QMV_EHIP: return "HIP error";
    default: return "unknown status";
    }
}

static qmv_status single(int t, const void *blocks, int64_t M, int64_t K, const float *x,
                         float *y, hipStream_t stream) {
    qmv_status st = check_matrix(t, blocks, M, K);
    if (st != QMV_OK) return st;
    if (!x || !y) return QMV_EINVAL;
    if (!aligned(x, 4) || !aligned(y, 4)) return QMV_EALIGN;
    SegTable seg{};
    seg.n = 1;
    seg.start[0] = 0;
    seg.start[1] = (int32_t)M;
    seg.y[0] = y;
    return from_hip(launch_rows_store(t, (const uint8_t *)blocks, M, K, x, seg, stream));
}

qmv_status qmv_q8_0(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream) {
    return single(kQ80, blocks, M, K, x, y, stream);
}
qmv_status qmv_q4_k(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream) {
    return single(kQ4K, blocks, M, K, x, y, stream);
}
qmv_status qmv_q6_k(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream) {
    return single(kQ6K, blocks, M, K, x, y, stream);
}
qmv_status qmv_q5_k(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream) {
    return single(kQ5K, blocks, M, K, x, y, stream);
}
qmv_status qmv_q2_k(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream) {
    return single(kQ2K, blocks, M, K, x, y, stream);
}
qmv_status qmv_q3_k(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream) {
    return single(kQ3K, blocks, M, K, x, y, stream);
}
qmv_status qmv_q4_0(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream) {
    return single(kQ40, blocks, M, K, x, y, stream);
}
qmv_status qmv_q4_1(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream) {
    return single(kQ41, blocks, M, K, x, y, stream);
}
qmv_status qmv_q5_0(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream) {
    return single(kQ50, blocks, M, K, x, y, stream);
}
qmv_status qmv_q5_1(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream) {
    return single(kQ51, blocks, M, K, x, y, stream);
}
qmv_status qmv_q8_1(const void *blocks, int64_t M, int64_t K, const float *x, float *y,
                    hipStream_t stream) {
    return single(kQ81, blocks, M, K, x, y, stream);
}

// Segment table of one row stack; total rows in *total.
static qmv_status build_segments(int32_t nseg, const int64_t *seg_rows, float *const *y_seg,
                                 SegTable &seg, int64_t *total_out) {
    if (!seg_rows || !y_seg) return QMV_EINVAL;
    if (nseg < 1 || nseg > QMV_MAX_SEGMENTS) return QMV_EINVAL;
    seg = SegTable{};
    seg.n = nseg;
    int64_t total = 0;
    for (int s = 0; s < nseg; s++) {
        if (seg_rows[s] < 1) return QMV_ESHAPE;
        if (!y_seg[s]) return QMV_EINVAL;
        if (!aligned(y_seg[s], 4)) return QMV_EALIGN;
        if (seg_rows[s] > 0x7FFFFFFFll - total) return QMV_ESHAPE;
        seg.start[s] = (int32_t)total;
        seg.y[s] = y_seg[s];
        total += seg_rows[s];
    }
    seg.start[nseg] = (int32_t)total;
    *total_out = total;
    return QMV_OK;
}

qmv_status qmv_fused_rows2(qmv_type t1, const void *blocks1, int32_t nseg1,
                           const int64_t *seg_rows1, float *const *y_seg1, qmv_type t2,
                           const void *blocks2, int32_t nseg2, const int64_t *seg_rows2,
                           float *const *y_seg2, int64_t K, const float *x, hipStream_t stream) {
    auto mixable = [](int t) { return t == kQ4K || t == kQ5K || t == kQ6K; };
    if (!mixable(t1) || !mixable(t2) || t1 == t2) return QMV_EINVAL;
    SegTable seg1, seg2;
    int64_t M1 = 0, M2 = 0;
    qmv_status st = build_segments(nseg1, seg_rows1, y_seg1, seg1, &M1);
    if (st != QMV_OK) return st;
    st = build_segments(nseg2, seg_rows2, y_seg2, seg2, &M2);
    if (st != QMV_OK) return st;
    st = check_matrix(t1, blocks1, M1, K);
    if (st != QMV_OK) return st;
    st = check_matrix(t2, blocks2, M2, K);
    if (st != QMV_OK) return st;
    if (!x) return QMV_EINVAL;
    if (!aligned(x, 4)) return QMV_EALIGN;
    return from_hip(launch_rows_mixed(t1, (const uint8_t *)blocks1, M1, seg1, t2,
                                      (const uint8_t *)blocks2, M2, seg2, K, x, stream));
}

qmv_status qmv_fused_rows(qmv_type t, const void *blocks, int64_t K, const float *x,
                          int32_t nseg, const int64_t *seg_rows, float *const *y_seg,
                          hipStream_t stream) {
    SegTable seg;
    int64_t total = 0;
    qmv_status st = build_segments(nseg, seg_rows, y_seg, seg, &total);
    if (st != QMV_OK) return st;
    st = check_matrix(t, blocks, total, K);
    if (st != QMV_OK) return st;
    if (!x) return QMV_EINVAL;
    if (!aligned(x, 4)) return QMV_EALIGN;
    return from_hip(launch_rows_store(t, (const uint8_t *)blocks, total, K, x, seg, stream));
}

qmv_status qmv_gate_up_silu(qmv_type t, const void *blocks, int64_t I, int64_t K, const float *x,
                            float *h, hipStream_t stream) {
    if (I < 1 || I > 0x3FFFFFFFll) return QMV_ESHAPE;
    qmv_status st = check_matrix(t, blocks, 2 * I, K);
    if (st != QMV_OK) return st;
    // the up row of a gate row is addressed by a 32-bit byte offset
    if ((uint64_t)I * row_bytes_of(t, K) > 0x7FFFFFFFull) return QMV_ESHAPE;
    if (!x || !h) return QMV_EINVAL;
    if (!aligned(x, 4) || !aligned(h, 4)) return QMV_EALIGN;
    return from_hip(launch_rows_silu(t, (const uint8_t *)blocks, I, K, x, h, stream));
}

qmv_status qmv_short_conv(qmv_type in_t, const void *in_proj, int64_t D, int64_t H, const float *h,
                          const float *w_conv, float *state, qmv_type out_t, const void *out_proj,
                          float *out, void *workspace, size_t ws_bytes, hipStream_t stream) {
    if (D < 1 || D > 0x1FFFFFFFll) return QMV_ESHAPE;
    qmv_status st = check_matrix(in_t, in_proj, 3 * D, H);
    if (st != QMV_OK) return st;
    st = check_matrix(out_t, out_proj, H, D);
    if (st != QMV_OK) return st;
    // the x row of a channel is 2D rows past its B row (32-bit byte offset)
    if ((uint64_t)2 * D * row_bytes_of(in_t, H) > 0x7FFFFFFFull) return QMV_ESHAPE;
    if (!h || !w_conv || !state || !out) return QMV_EINVAL;
    if (!aligned(h, 4) || !aligned(w_conv, 4) || !aligned(state, 4) || !aligned(out, 4))
        return QMV_EALIGN;
    if (!workspace || ws_bytes < qmv_workspace_bytes(QMV_OP_SHORT_CONV, D, 0, 0, 0))
        return QMV_EWORKSPACE;
    if (!aligned(workspace, 16)) return QMV_EALIGN;
    return from_hip(launch_short_conv(in_t, (const uint8_t *)in_proj, D, H, h, w_conv, state, out_t,
                                      (const uint8_t *)out_proj, out, (float *)workspace, stream));
}

qmv_status qmv_argmax(qmv_type t, const void *blocks, int64_t M, int64_t K, const float *x,
                      int32_t *idx_out, float *max_out, void *workspace, size_t ws_bytes,
                      hipStream_t stream) {
    qmv_status st = check_matrix(t, blocks, M, K);
    if (st != QMV_OK) return st;
    if (!x || !idx_out || !max_out) return QMV_EINVAL;
    if (!aligned(x, 4) || !aligned(idx_out, 4) || !aligned(max_out, 4)) return QMV_EALIGN;
    if (!workspace || ws_bytes < qmv_workspace_bytes(QMV_OP_ARGMAX, M, K, 0, 0))
        return QMV_EWORKSPACE;
    if (!aligned(workspace, 8)) return QMV_EALIGN;
    return from_hip(launch_rows_argmax(t, (const uint8_t *)blocks, M, K, x,
                                       (uint64_t *)workspace, idx_out, max_out, stream));
}

qmv_status qmv_argmax_noalloc(qmv_type t, const void *blocks, int64_t M, int64_t K,
                              const float *x, int32_t *idx_out, float *max_out,
                              hipStream_t stream) {
    qmv_status st = check_matrix(t, blocks, M, K);
    if (st != QMV_OK) return st;
    if (!x || !idx_out || !max_out) return QMV_EINVAL;
    if (!aligned(x, 4) || !aligned(idx_out, 4) || !aligned(max_out, 4)) return QMV_EALIGN;
    return from_hip(launch_rows_argmax_noalloc(t, (const uint8_t *)blocks, M, K, x, idx_out,
                                               max_out, stream));
}

qmv_status moe_qmv_topk(const float *x, int64_t H, const float *router, const float *bias,
                        int32_t E, int32_t k, qmv_type gu_t, const void *gate_up,
                        qmv_type dn_t, const void *down, int64_t I, float *y,
                        int32_t *topk_idx, float *topk_w, void *workspace, size_t ws_bytes,
                        hipStream_t stream) {
    if (!x || !router || !bias || !gate_up || !down || !y || !topk_idx || !topk_w)
        return QMV_EINVAL;
    if (!valid_type(gu_t) || !valid_type(dn_t)) return QMV_EINVAL;
    if (E < 1 || E > 64 || k < 1 || k > E) return QMV_ESHAPE;
    if (H < 1 || I < 1 || (int64_t)k * I > QMV_MAX_K || (int64_t)k * 2 * I > 0x7FFFFFFFll)
        return QMV_ESHAPE;
    if (block_weights_of(dn_t) == 32 && I % 128 != 0) return QMV_ESHAPE;
    qmv_status st = check_matrix(gu_t, gate_up, 2 * I, H);
    if (st != QMV_OK) return st;
    st = check_matrix(dn_t, down, H, I);
    if (st != QMV_OK) return st;
    if (!aligned(x, 4) || !aligned(router, 4) || !aligned(bias, 4) || !aligned(y, 4) ||
        !aligned(topk_idx, 4) || !aligned(topk_w, 4))
        return QMV_EALIGN;
    if (!workspace || ws_bytes < qmv_workspace_bytes(QMV_OP_MOE, H, I, E, k))
        return QMV_EWORKSPACE;
    if (!aligned(workspace, 16)) return QMV_EALIGN;
    return from_hip(launch_moe(x, H, router, bias, E, k, gu_t, (const uint8_t *)gate_up, dn_t,
                               (const uint8_t *)down, I, y, topk_idx, topk_w,
                               (uint8_t *)workspace, stream));
}

qmv_status qmv_gemm_n(qmv_type t, const void *blocks, int64_t M, int64_t K, int32_t n,
                      const float *X, float *Y, void *workspace, size_t ws_bytes,
                      hipStream_t stream) {
    if (!mfma_type(t)) return QMV_EINVAL;
    qmv_status st = check_matrix(t, blocks, M, K);
    if (st != QMV_OK) return st;
    if (n < 1 || n > QMV_MAX_N) return QMV_ESHAPE;
    if (!X || !Y) return QMV_EINVAL;
    if (!aligned(X, 4) || !aligned(Y, 4)) return QMV_EALIGN;
    const size_t need = gemm_n_workspace(M, K, n);
    if (need > 0 && (!workspace || ws_bytes < need)) return QMV_EWORKSPACE;
    if (need > 0 && !aligned(workspace, 16)) return QMV_EALIGN;
    return from_hip(launch_gemm_n(t, (const uint8_t *)blocks, M, K, n, X, Y, workspace, stream));
}

qmv_status qmv_gemm(qmv_type t, const void *blocks, int64_t M, int64_t K, int64_t n, const float *X,
                    float *Y, void *workspace, size_t ws_bytes, hipStream_t stream) {
    if (!mfma_type(t)) return QMV_EINVAL;
    qmv_status st = check_matrix(t, blocks, M, K);
    if (st != QMV_OK) return st;
    if (n < 1 || n > QMV_MAX_PREFILL_N) return QMV_ESHAPE;
    // X is addressed with 32-bit byte offsets
    if ((uint64_t)n * (uint64_t)K * 4u > 0xFFFFFFFFull) return QMV_ESHAPE;
    if (!X || !Y) return QMV_EINVAL;
    if (!aligned(X, 4) || !aligned(Y, 4)) return QMV_EALIGN;
    const size_t need = gemm_workspace(M, K, n);
    if (need > 0) {
        if (!workspace || ws_bytes < need) return QMV_EWORKSPACE;
        if (!aligned(workspace, 16)) return QMV_EALIGN;
    }
    return from_hip(launch_gemm(t, (const uint8_t *)blocks, M, K, n, X, Y, workspace, stream));
}

qmv_status qmv_dequant(qmv_type t, const void *blocks, int64_t M, int64_t K, float *w_out,
                       hipStream_t stream) {
    qmv_status st = check_matrix(t, blocks, M, K);
    if (st != QMV_OK) return st;
    if (!w_out) return QMV_EINVAL;
    if (!aligned(w_out, 16)) return QMV_EALIGN;
    return from_hip(launch_dequant(t, (const uint8_t *)blocks, M, K, w_out, stream));
}

qmv_status qmv_quantize(qmv_type t, const float *w, int64_t M, int64_t K, void *blocks_out,
                        hipStream_t stream) {
    if (!core_type(t)) return QMV_EINVAL;
    if (!w || !blocks_out) return QMV_EINVAL;
    if (M < 1 || K < 1 || K > QMV_MAX_K || K % block_weights_of(t) != 0) return QMV_ESHAPE;
    if (M > 0x7FFFFFFFll) return QMV_ESHAPE;
    if (!aligned(w, 4)) return QMV_EALIGN;
    return from_hip(launch_quantize(t, w, M, K, (uint8_t *)blocks_out, stream));
}

qmv_status qmv_time_next_launch(hipEvent_t start, hipEvent_t stop) {
    if ((start == nullptr) != (stop == nullptr)) return QMV_EINVAL;
    set_timing_hook(start, stop);
    return QMV_OK;
}

qmv_status qmv_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink,
                                 hipStream_t stream) {
    if (!buf || !sink || bytes == 0 || bytes % 16 != 0) return QMV_EINVAL;
    if (!aligned(buf, 16) || !aligned(sink, 4)) return QMV_EALIGN;
    return from_hip(launch_probe(buf, bytes, sink, stream));
}

}  // extern "C"
