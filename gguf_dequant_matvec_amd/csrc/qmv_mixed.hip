// Fused rows over two row stacks of different block formats in one launch
// (FlareLLM page, section "推理层面的深度优化": fused QKV; BebeLM page,
// section "量化格式支持": Q4_K_M keeps the attention V projection in Q6_K
// while Q and K are Q4_K).
#include "qmv_launch.h"

namespace qmv {

namespace {

using Kernel2 = void (*)(RowsParams, RowsParams, int);

template <class F1, class F2, bool XR>
Kernel2 mixed_for(int G) {
    switch (G) {
    case 4: return rows2_kernel<F1, F2, 4, XR>;
    case 8: return rows2_kernel<F1, F2, 8, XR>;
    case 16: return rows2_kernel<F1, F2, 16, XR>;
    case 32: return rows2_kernel<F1, F2, 32, XR>;
    default: return rows2_kernel<F1, F2, 64, XR>;
    }
}

// Both formats have 64-weight units, so the lane group G (a function of the
// unit count per row) is the one each stack's own launch would use, and every
// row's result is bit-identical to that launch's.  The workgroups are split
// between the stacks in proportion to their tiles when both do not fit.
template <class F1, class F2>
hipError_t launch_mixed_typed(const RowsParams &p1, const RowsParams &p2, hipStream_t s) {
    static_assert(F1::kUnitWeights == F2::kUnitWeights, "same unit size");
    const int U = p1.K / F1::kUnitWeights;
    const int G = pick_group(U);
    const int iters = (U + G - 1) / G;
    const int64_t rows_per_tile = (int64_t)kR * (kWave / G);
    const int64_t nt1 = (p1.M + rows_per_tile - 1) / rows_per_tile;
    const int64_t nt2 = (p2.M + rows_per_tile - 1) / rows_per_tile;
    const int waves = kBlockThreads / kWave;
    const size_t l1 = ((size_t)lds_x_floats<F1>(p1.K) + (size_t)p1.K / F1::kSumGroup) * 4;
    const size_t l2 = ((size_t)lds_x_floats<F2>(p2.K) + (size_t)p2.K / F2::kSumGroup) * 4;
    const size_t lds = l1 > l2 ? l1 : l2;
    Kernel2 k = iters == 1 ? mixed_for<F1, F2, true>(G) : mixed_for<F1, F2, false>(G);
    hipError_t e = ensure_lds((const void *)k, lds);
    if (e != hipSuccess) return e;
    int per_cu = resident_blocks((const void *)k, kBlockThreads, lds);
    if (per_cu > kMaxBlocksPerCU) per_cu = kMaxBlocksPerCU;
    const int64_t cap = (int64_t)device_cu_count() * per_cu;
    int64_t g1 = (nt1 + waves - 1) / waves, g2 = (nt2 + waves - 1) / waves;
    if (g1 + g2 > cap) {
        g1 = (cap * nt1 + (nt1 + nt2) / 2) / (nt1 + nt2);
        if (g1 < 1) g1 = 1;
        if (g1 > cap - 1) g1 = cap - 1;
        g2 = cap - g1;
    }
    return launch_main(k, dim3((unsigned)(g1 + g2)), dim3(kBlockThreads), lds, s, p1, p2, (int)g1);
}

}  // namespace

hipError_t launch_rows_mixed(int t1, const uint8_t *W1, int64_t M1, const SegTable &seg1, int t2,
                             const uint8_t *W2, int64_t M2, const SegTable &seg2, int64_t K,
                             const float *x, hipStream_t s) {
    RowsParams p1{}, p2{};
    p1.W = W1;
    p1.M = (int32_t)M1;
    p1.seg = seg1;
    p2.W = W2;
    p2.M = (int32_t)M2;
    p2.seg = seg2;
    for (RowsParams *p : {&p1, &p2}) {
        p->K = (int32_t)K;
        p->x = x;
        p->partials = nullptr;
    }
    p1.row_bytes = (int64_t)row_bytes_of(t1, K);
    p2.row_bytes = (int64_t)row_bytes_of(t2, K);
    // canonical order of the format pair (the caller's order is kept in the
    // parameters, so only the kernel choice depends on it)
    if (t1 > t2) return launch_rows_mixed(t2, W2, M2, seg2, t1, W1, M1, seg1, K, x, s);
    if (t1 == kQ4K && t2 == kQ5K) return launch_mixed_typed<Q4K, Q5K>(p1, p2, s);
    if (t1 == kQ4K && t2 == kQ6K) return launch_mixed_typed<Q4K, Q6K>(p1, p2, s);
    if (t1 == kQ5K && t2 == kQ6K) return launch_mixed_typed<Q5K, Q6K>(p1, p2, s);
    return hipErrorInvalidValue;
}

}  // namespace qmv
