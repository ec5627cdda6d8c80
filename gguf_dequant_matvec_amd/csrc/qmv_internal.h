// Host-side declarations shared by the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>

namespace qmv {

struct SegTable;

enum {
    kQ40 = 2, kQ41 = 3, kQ50 = 6, kQ51 = 7, kQ80 = 8, kQ81 = 9,
    kQ2K = 10, kQ3K = 11, kQ4K = 12, kQ5K = 13, kQ6K = 14
};

constexpr int kMaxGrid = 2048;  // largest persistent grid (argmax partial slots)

inline int block_weights_of(int type) {
    switch (type) {
    case kQ40: case kQ41: case kQ50: case kQ51: case kQ80: case kQ81: return 32;
    case kQ2K: case kQ3K: case kQ4K: case kQ5K: case kQ6K: return 256;
    default: return 0;
    }
}
inline int block_bytes_of(int type) {
    switch (type) {
    case kQ40: return 18;
    case kQ41: return 20;
    case kQ50: return 22;
    case kQ51: return 24;
    case kQ80: return 34;
    case kQ81: return 36;
    case kQ2K: return 84;
    case kQ3K: return 110;
    case kQ4K: return 144;
    case kQ5K: return 176;
    case kQ6K: return 210;
    default: return 0;
    }
}
inline size_t row_bytes_of(int type, int64_t K) {
    const int bw = block_weights_of(type);
    return bw ? (size_t)(K / bw) * (size_t)block_bytes_of(type) : 0;
}

// One-shot kernel timing hook of the calling thread (see qmv_time_next_launch).
struct TimingHook {
    hipEvent_t start = nullptr, stop = nullptr;
};
void set_timing_hook(hipEvent_t start, hipEvent_t stop);
TimingHook take_timing_hook();

// Enqueue `kernel` and return the status of this enqueue itself (not a
// sticky error left by an earlier call): the arguments are converted to the
// kernel's parameter types and passed by address to hipLaunchKernel, or to
// hipExtLaunchKernel when timing events are given.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                         hipStream_t s, hipEvent_t start, hipEvent_t stop, Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    std::tuple<typename std::decay<KArgs>::type...> vals(args...);
    void *argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
    std::apply([&](auto &...v) {
        int i = 0;
        ((argv[i++] = (void *)&v), ...);
    }, vals);
    if (start && stop)
        return hipExtLaunchKernel((const void *)kernel, grid, block, argv, lds, s, start, stop, 0);
    return hipLaunchKernel((const void *)kernel, grid, block, argv, lds, s);
}

// Launch a call's main kernel, with the thread's timing events when the hook
// is armed (the hook is consumed).
template <typename Kernel, typename... Args>
hipError_t launch_main(Kernel kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                       Args... args) {
    TimingHook h = take_timing_hook();
    return launch_kernel(kernel, grid, block, lds, s, h.start, h.stop, args...);
}

// Launch a helper kernel of a call (never timed).
template <typename Kernel, typename... Args>
hipError_t launch_aux(Kernel kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                      Args... args) {
    return launch_kernel(kernel, grid, block, lds, s, nullptr, nullptr, args...);
}

// Compute units of the current device (cached per device).
int device_cu_count();
// Workgroups of `kernel` that can be resident on one compute unit at once
// (occupancy query, cached per kernel and LDS size; at least 1).
int resident_blocks(const void *kernel, int threads, size_t lds);
// Raise a kernel's dynamic-LDS limit when it needs more than the default.
hipError_t ensure_lds(const void *kernel, size_t bytes);

hipError_t launch_rows_store(int type, const uint8_t *W, int64_t M, int64_t K, const float *x,
                             const SegTable &seg, hipStream_t s);
hipError_t launch_rows_mixed(int t1, const uint8_t *W1, int64_t M1, const SegTable &seg1, int t2,
                             const uint8_t *W2, int64_t M2, const SegTable &seg2, int64_t K,
                             const float *x, hipStream_t s);
hipError_t launch_rows_silu(int type, const uint8_t *W, int64_t I, int64_t K, const float *x,
                            float *h, hipStream_t s);
hipError_t launch_short_conv(int in_t, const uint8_t *in_proj, int64_t D, int64_t H,
                             const float *h, const float *w_conv, float *state, int out_t,
                             const uint8_t *out_proj, float *out, float *y, hipStream_t s);
hipError_t launch_rows_argmax(int type, const uint8_t *W, int64_t M, int64_t K, const float *x,
                              uint64_t *partials, int32_t *idx_out, float *max_out,
                              hipStream_t s);
// qmv_argmax with its per-workgroup keys in a device-global array.
hipError_t launch_rows_argmax_noalloc(int type, const uint8_t *W, int64_t M, int64_t K,
                                      const float *x, int32_t *idx_out, float *max_out,
                                      hipStream_t s);
hipError_t launch_dequant(int type, const uint8_t *W, int64_t M, int64_t K, float *out,
                          hipStream_t s);
hipError_t launch_quantize(int type, const float *w, int64_t M, int64_t K, uint8_t *out,
                           hipStream_t s);
hipError_t launch_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s);
hipError_t launch_moe(const float *x, int64_t H, const float *router, const float *bias,
                      int32_t E, int32_t k, int gu_t, const uint8_t *gate_up, int dn_t,
                      const uint8_t *down, int64_t I, float *y, int32_t *topk_idx,
                      float *topk_w, uint8_t *ws, hipStream_t s);
// Prefill product plan: tokens per workgroup (16 tt), 16-row tiles per wave
// (rt), token blocks, padded row groups, K slices and windows per slice.
struct PfPlan {
    int tt, rt, token_blocks, rg_pad, slices, wps;
};
PfPlan pf_plan(int64_t M, int64_t K, int64_t n);
size_t gemm_workspace(int64_t M, int64_t K, int64_t n);
hipError_t launch_gemm(int type, const uint8_t *W, int64_t M, int64_t K, int64_t n, const float *X,
                       float *Y, void *ws, hipStream_t s);
hipError_t launch_gemm_n(int type, const uint8_t *W, int64_t M, int64_t K, int32_t n,
                         const float *X, float *Y, void *ws, hipStream_t s);
size_t gemm_n_workspace(int64_t M, int64_t K, int32_t n);
// Y[t][i] = sum over K slices of partial[slice][t][i] (nm = n * M outputs), in
// slice order: the second launch of K-split products.
hipError_t launch_slice_reduce(const float *partial, int slices, int64_t nm, float *Y,
                               hipStream_t s);

}  // namespace qmv
