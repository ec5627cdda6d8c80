// Definition of the row-kernel launcher (kernel choice, grid and LDS size per
// call).  Included only by qmv_rows_inst.hip, which instantiates it once per
// (format, mode).
#pragma once

#include "qmv_launch.h"

namespace qmv {

template <class F, int MODE, int KS, bool XR, int R = rows_per_lane<MODE>(),
          int BT = kBlockThreads>
KernelPtr<F, MODE> kernel_for_ks(int G) {
    switch (G) {
    case 4: return rows_kernel<F, 4, R, MODE, KS, XR, BT>;
    case 8: return rows_kernel<F, 8, R, MODE, KS, XR, BT>;
    case 16: return rows_kernel<F, 16, R, MODE, KS, XR, BT>;
    case 32: return rows_kernel<F, 32, R, MODE, KS, XR, BT>;
    default: return rows_kernel<F, 64, R, MODE, KS, XR, BT>;
    }
}

template <class F, int MODE>
hipError_t launch_typed(const RowsParams &p_in, hipStream_t s, int *grid_out) {
    RowsParams p = p_in;
    if (MODE == kModeMoeDown) p.moe.units_per_mat = p.moe.I / F::kUnitWeights;
    const int U = p.K / F::kUnitWeights;
    // the MoE down launch needs unit steps that never straddle two experts
    const int G = MODE == kModeMoeDown ? pow2_divisor(p.moe.units_per_mat) : pick_group(U);
    const int iters = (U + G - 1) / G;
    // Plain launches with long rows (K >= 8192: x of 32 KB or more, staged in
    // LDS) use one 8-wave workgroup per compute unit instead of two 4-wave
    // ones, so each compute unit stages x once, not twice (4096 x 14336
    // Q4_K: 11.4 -> 9.9 us).  Shorter rows keep two 4-wave workgroups
    // (gate+up 28672 x 4096 was slower with one 8-wave, and Q8_0 1536 x 576
    // went from 4.2 to 5.7 us with half as many workgroups); so do the
    // formats that keep two (keeps_two_workgroups).
    const bool wide = MODE == kModeStore && iters > 1 && p.K >= 8192 && !keeps_two_workgroups<F>();
    const int bt = wide ? kWideBlockThreads : kBlockThreads;
    const int waves = bt / kWave;
    const int64_t total_waves =
        (int64_t)device_cu_count() * kMaxBlocksPerCU * (kBlockThreads / kWave);
    // Plain and argmax launches take one row slot instead of two when two
    // would leave at most one tile per wave of a full grid (no next item to
    // overlap), always for the argmax (its vocabulary-sized matrix ran 6%
    // faster with one) and always for the formats that prefer one.  Row
    // slots do not change any row's arithmetic.
    constexpr bool kOneSlotModes = MODE == kModeStore || MODE == kModeArgmax;
    bool one_slot = false;
    if (kOneSlotModes) {
        const int64_t tiles2 = ((int64_t)p.M + 2 * (kWave / G) - 1) / (2 * (kWave / G));
        one_slot = MODE == kModeArgmax || prefers_one_slot<F>() || tiles2 <= total_waves;
    }
    // stacked modes: the row slots hold rows M apart (gate/up; B/C/x)
    const int64_t rows_per_tile =
        (MODE == kModeSiluUp || MODE == kModeShortConv || MODE == kModeMoeGateUp || one_slot ? 1
                                                                   : (int64_t)rows_per_lane<MODE>()) *
        (kWave / G);
    const int64_t ntiles = ((int64_t)p.M + rows_per_tile - 1) / rows_per_tile;
    const size_t lds =
        ((size_t)lds_x_floats<F>(p.K) + (F::kSumGroup ? (size_t)p.K / F::kSumGroup : 0)) * 4;
    // Tiles of one wave each.  The MoE down launch (few rows, long rows)
    // splits each tile's K over the 4 waves of a workgroup when it has fewer
    // than two tiles per compute unit and at least 4 unit steps per row.  The
    // other modes never split, so a row's result depends only on (format, K)
    // and fused rows and the argmax stay bit-identical to the plain matvec.
    // a row of one unit step keeps its activations in registers
    constexpr bool kXrModes = MODE == kModeStore || MODE == kModeArgmax || MODE == kModeSiluUp ||
                              MODE == kModeShortConv || MODE == kModeMoeGateUp;
    KernelPtr<F, MODE> k = iters == 1 ? kernel_for_ks<F, MODE, 1, kXrModes>(G)
                                      : kernel_for_ks<F, MODE, 1, false>(G);
    if constexpr (kOneSlotModes) {
        if (one_slot)
            k = iters == 1 ? kernel_for_ks<F, MODE, 1, kXrModes, 1>(G)
                           : kernel_for_ks<F, MODE, 1, false, 1>(G);
    }
    if constexpr (MODE == kModeStore) {
        if (wide)
            k = one_slot ? kernel_for_ks<F, MODE, 1, false, 1, kWideBlockThreads>(G)
                         : kernel_for_ks<F, MODE, 1, false, kR, kWideBlockThreads>(G);
    }
    hipError_t e = ensure_lds((const void *)k, lds);
    if (e != hipSuccess) return e;
    int per_cu = resident_blocks((const void *)k, bt, lds);
    const bool split = MODE == kModeMoeDown && iters >= waves &&
                       ntiles < 2 * (int64_t)device_cu_count();
    if (split) {
        k = kernel_for_ks<F, MODE, MODE == kModeMoeDown ? kBlockThreads / kWave : 1, false>(G);
        e = ensure_lds((const void *)k, lds);
        if (e != hipSuccess) return e;
        per_cu = resident_blocks((const void *)k, kBlockThreads, lds);
    }
    // Each workgroup stages its own copy of x, and the x loads of a compute
    // unit's later workgroups queue behind the earlier ones' first weight
    // loads: with three or more workgroups per compute unit the last ones
    // start late and end the launch late, so at most two are used (measured
    // faster at every decode shape).
    if (per_cu > kMaxBlocksPerCU) per_cu = kMaxBlocksPerCU;
    if (wide) per_cu = 1;
    // persistent grid: at most the workgroups that are resident at once, so
    // no workgroup waits for a second round while compute units idle
    int64_t grid = split ? ntiles : (ntiles + waves - 1) / waves;
    const int64_t cap = (int64_t)device_cu_count() * per_cu;
    if (grid > cap) grid = cap;
    if (grid > kMaxGrid) grid = kMaxGrid;
    if (grid < 1) grid = 1;
    if (grid_out) *grid_out = (int)grid;
    return launch_main(k, dim3((unsigned)grid), dim3((unsigned)bt), lds, s, p);
}

}  // namespace qmv
