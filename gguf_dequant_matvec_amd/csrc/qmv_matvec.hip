// Single-token, fused-row and argmax launches of the row-streaming kernel.
#include "qmv_launch.h"

namespace qmv {

namespace {

__global__ __launch_bounds__(256) void argmax_finalize(const uint64_t *partials, int n,
                                                       int32_t *idx_out, float *max_out) {
    __shared__ uint64_t red[256];
    uint64_t k = 0;
    for (int i = threadIdx.x; i < n; i += 256) k = partials[i] > k ? partials[i] : k;
    red[threadIdx.x] = k;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) {
            const uint64_t b = red[threadIdx.x + o];
            red[threadIdx.x] = b > red[threadIdx.x] ? b : red[threadIdx.x];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const uint64_t best = red[0];
        *idx_out = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
        *max_out = key_float((uint32_t)(best >> 32));
    }
}

}  // namespace

hipError_t launch_rows_store(int type, const uint8_t *W, int64_t M, int64_t K, const float *x,
                             const SegTable &seg, hipStream_t s) {
    RowsParams p{};
    p.W = W;
    p.M = (int32_t)M;
    p.K = (int32_t)K;
    p.row_bytes = (int64_t)row_bytes_of(type, K);
    p.x = x;
    p.seg = seg;
    p.partials = nullptr;
    return launch_fmt<kModeStore>(type, p, s, nullptr);
}

hipError_t launch_rows_argmax(int type, const uint8_t *W, int64_t M, int64_t K, const float *x,
                              uint64_t *partials, int32_t *idx_out, float *max_out,
                              hipStream_t s) {
    RowsParams p{};
    p.W = W;
    p.M = (int32_t)M;
    p.K = (int32_t)K;
    p.row_bytes = (int64_t)row_bytes_of(type, K);
    p.x = x;
    p.seg.n = 0;
    p.partials = partials;
    int grid = 0;
    hipError_t e = launch_fmt<kModeArgmax>(type, p, s, &grid);
    if (e != hipSuccess) return e;
    return launch_aux(argmax_finalize, dim3(1), dim3(256), 0, s, (const uint64_t *)partials, grid,
                      idx_out, max_out);
}

}  // namespace qmv
