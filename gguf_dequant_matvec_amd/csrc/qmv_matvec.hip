// Single-token, fused-row and argmax launches of the row-streaming kernel.
#include "qmv_internal.h"
#include "qmv_rows.h"

namespace qmv {

namespace {

// Fraction of lane-steps that carry work when a row of U units is spread over
// G lanes; the launcher picks the G (>= 4, a power of two) that maximises it,
// preferring wider groups on ties (fewer rows per wave, better coalescing).
int pick_group(int U) {
    int best = 64;
    double best_eff = -1.0;
    for (int G = 64; G >= 4; G >>= 1) {
        const int steps = (U + G - 1) / G;
        const double eff = (double)U / ((double)G * steps);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best = G;
        }
    }
    return best;
}

constexpr int kR = 2;  // row slots per lane

template <class F, int MODE>
using KernelPtr = void (*)(RowsParams);

template <class F, int MODE>
KernelPtr<F, MODE> kernel_for(int G) {
    switch (G) {
    case 4: return rows_kernel<F, 4, kR, MODE>;
    case 8: return rows_kernel<F, 8, kR, MODE>;
    case 16: return rows_kernel<F, 16, kR, MODE>;
    case 32: return rows_kernel<F, 32, kR, MODE>;
    default: return rows_kernel<F, 64, kR, MODE>;
    }
}

template <class F, int MODE>
hipError_t launch_typed(const RowsParams &p, hipStream_t s, int *grid_out) {
    const int U = p.K / F::kUnitWeights;
    const int G = pick_group(U);
    const int64_t rows_per_tile = (int64_t)kR * (kWave / G);
    const int64_t ntiles = ((int64_t)p.M + rows_per_tile - 1) / rows_per_tile;
    const int waves = kBlockThreads / kWave;
    const size_t lds =
        ((size_t)lds_x_floats<F>(p.K) + (F::kSumGroup ? (size_t)p.K / F::kSumGroup : 0)) * 4;
    KernelPtr<F, MODE> k = kernel_for<F, MODE>(G);
    hipError_t e = ensure_lds((const void *)k, lds);
    if (e != hipSuccess) return e;
    // persistent grid: exactly the workgroups that are resident at once, so
    // no workgroup waits for a second round while compute units idle
    const int per_cu = resident_blocks((const void *)k, kBlockThreads, lds);
    int64_t grid = (ntiles + waves - 1) / waves;
    const int64_t cap = (int64_t)device_cu_count() * per_cu;
    if (grid > cap) grid = cap;
    if (grid > kMaxGrid) grid = kMaxGrid;
    if (grid < 1) grid = 1;
    if (grid_out) *grid_out = (int)grid;
    return launch_main(k, dim3((unsigned)grid), dim3(kBlockThreads), lds, s, p);
}

template <int MODE>
hipError_t launch_fmt(int type, const RowsParams &p, hipStream_t s, int *grid_out) {
    switch (type) {
    case kQ4K: return launch_typed<Q4K, MODE>(p, s, grid_out);
    case kQ6K: return launch_typed<Q6K, MODE>(p, s, grid_out);
    case kQ80:
        if ((p.K / 32) % 2 == 0) return launch_typed<Q80x2, MODE>(p, s, grid_out);
        return launch_typed<Q80x1, MODE>(p, s, grid_out);
    default: return hipErrorInvalidValue;
    }
}

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
    hipLaunchKernelGGL(argmax_finalize, dim3(1), dim3(256), 0, s, partials, grid, idx_out,
                       max_out);
    return hipGetLastError();
}

}  // namespace qmv
