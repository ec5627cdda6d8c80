// Single-token, fused-row and argmax launches of the row-streaming kernel.
#include "qmv.h"
#include "qmv_launch.h"

#include <mutex>

namespace qmv {

namespace {

// Scratch of qmv_argmax_noalloc: the per-workgroup (value, index) keys of one
// argmax launch, whose grid never exceeds kMaxGrid workgroups.  A device
// global (16 KiB), so every GPU the library runs on holds its own copy until
// the process ends and no call allocates.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels get the device address that
// hipGetSymbolAddress returns for the current device (scratch_of_device).
__device__ __align__(256) uint64_t scratch[kMaxGrid];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mutex;
uint64_t *g_scratch_ptr[kScratchDevices];

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

// Device address of this device's scratch array, looked up once per device
// (with that device current) and kept.
static hipError_t scratch_of_device(uint64_t **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<uint64_t *>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_rows_argmax_noalloc(int type, const uint8_t *W, int64_t M, int64_t K,
                                      const float *x, int32_t *idx_out, float *max_out,
                                      hipStream_t s) {
    // the argmax launch caps its grid at kMaxGrid, one key per workgroup
    static_assert(sizeof(scratch) == (size_t)kMaxGrid * sizeof(uint64_t), "one key per workgroup");
    static_assert(kMaxGrid == QMV_ARGMAX_SCRATCH_KEYS, "the documented scratch size");
    uint64_t *keys = nullptr;
    hipError_t e = scratch_of_device(&keys);
    if (e != hipSuccess) return e;
    return launch_rows_argmax(type, W, M, K, x, keys, idx_out, max_out, s);
}

}  // namespace qmv
