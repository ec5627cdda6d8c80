// Host-side launch helpers for the row-streaming kernel (one mode per
// translation unit instantiates its kernels).
#pragma once

#include "qmv_internal.h"
#include "qmv_rows.h"

#include <type_traits>

namespace qmv {

constexpr int kR = 2;  // row slots per lane
constexpr int kMaxBlocksPerCU = 2;  // persistent workgroups per compute unit

// Fraction of lane-steps that carry work when a row of U units is spread over
// G lanes; pick the G (a power of two, >= 4) that maximises it, preferring
// wider groups on ties (fewer rows per wave, better coalescing).
inline int pick_group(int U) {
    // Rows of 9-32 units take one step of 16 or 32 lanes (a wave's item
    // chain is then one item per tile and x stays in registers), even
    // though up to 44% of the lanes idle: matrices of such short rows are
    // small and latency-bound.  Measured (MI355X, cold, us): Q8_0 1536x576
    // 4.10 -> 3.02 (groups of 4, three steps, before), Q4_K 8192x768 4.10 ->
    // 3.56, Q4_K 1536x1536 4.0 -> 3.17 and 8960x1536 5.28 -> 5.13, Q6_K
    // 8960x1536 6.53 -> 5.80, Q8_0 8960x1536 6.2 -> 5.61, and 32768x576 no
    // slower (7.0 -> 6.8).  Longer rows keep the rule below: with 40 units
    // one 64-lane step made 20000x2560 slower (9.5 -> 10.1) though 2048x2560
    // faster (5.18 -> 3.82).
    if (U > 8 && U <= 32) return U <= 16 ? 16 : 32;
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

// Largest power of two <= 64 that divides n (n a multiple of 4).
inline int pow2_divisor(int n) {
    int G = 64;
    while (G > 4 && n % G != 0) G >>= 1;
    return G;
}

template <class F, int MODE>
using KernelPtr = void (*)(RowsParams);

// Row slots per lane: the MoE down launch has few rows (the hidden size)
// and long rows (k experts), so it keeps one slot for more tiles.
template <int MODE>
constexpr int rows_per_lane() {
    return MODE == kModeMoeDown ? 1 : MODE == kModeShortConv ? 3 : kR;
}

// Formats whose plain launches run faster with one row slot at every size
// (measured at 14336-128000 rows: Q6_K 15% faster, Q8_0 in two-block units
// 1.5%; every other format is 6-35% slower with one).
template <class F>
constexpr bool prefers_one_slot() {
    return std::is_same<F, Q6K>::value || std::is_same<F, Q80x2>::value;
}

// Formats whose plain launches with long rows keep two 4-wave workgroups per
// compute unit instead of one 8-wave one (measured for Q6_K, us: 14336 x
// 14336 36.8 -> 32.8, 4096 x 8192 8.79 -> 8.42, 2048 x 8192 6.65 -> 6.19,
// 4096 x 14336 13.0 either way; Q4_K was slower with two: 2048 x 8192 5.06
// -> 5.39, 4096 x 8192 7.1 -> 7.4; Q8_0 mixed: 14336 x 14336 39.1 -> 38.3,
// 4096 x 14336 13.4 -> 13.8).
template <class F>
constexpr bool keeps_two_workgroups() {
    return std::is_same<F, Q6K>::value;
}

// The launcher of the row kernel for one (format, mode).  Its definition
// lives in qmv_launch_impl.h and is instantiated once per (format, mode) in
// qmv_rows_inst.hip, so the kernels compile in parallel units.
template <class F, int MODE>
hipError_t launch_typed(const RowsParams &p_in, hipStream_t s, int *grid_out);

template <int MODE>
hipError_t launch_fmt(int type, const RowsParams &p, hipStream_t s, int *grid_out) {
    switch (type) {
    case kQ2K: return launch_typed<Q2K, MODE>(p, s, grid_out);
    case kQ3K: return launch_typed<Q3K, MODE>(p, s, grid_out);
    case kQ4K: return launch_typed<Q4K, MODE>(p, s, grid_out);
    case kQ5K: return launch_typed<Q5K, MODE>(p, s, grid_out);
    case kQ6K: return launch_typed<Q6K, MODE>(p, s, grid_out);
    case kQ40: case kQ41: case kQ50: case kQ51: case kQ81: {
        // one 32-weight block per unit; in the MoE down launch the units per
        // expert (I / 32) must be a multiple of the narrowest lane group (4)
        if (MODE == kModeMoeDown && (p.moe.I / 32) % 4 != 0) return hipErrorInvalidValue;
        // Q4_0, Q5_0, Q4_1 and Q5_1 take two blocks per unit when a row, or
        // in the MoE down launch an expert, holds an even number of blocks
        // (there: a multiple of four two-block units)
        const bool pair = MODE == kModeMoeDown ? p.moe.I % 64 == 0 && (p.moe.I / 64) % 4 == 0
                                               : (p.K / 32) % 2 == 0;
        switch (type) {
        case kQ40: return pair ? launch_typed<Q40x2, MODE>(p, s, grid_out) : launch_typed<Q40, MODE>(p, s, grid_out);
        case kQ41: return pair ? launch_typed<Q41x2, MODE>(p, s, grid_out) : launch_typed<Q41, MODE>(p, s, grid_out);
        case kQ50: return pair ? launch_typed<Q50x2, MODE>(p, s, grid_out) : launch_typed<Q50, MODE>(p, s, grid_out);
        case kQ51: return pair ? launch_typed<Q51x2, MODE>(p, s, grid_out) : launch_typed<Q51, MODE>(p, s, grid_out);
        default: return launch_typed<Q81x1, MODE>(p, s, grid_out);
        }
    }
    case kQ80:
        if (MODE == kModeMoeDown) {
            // unit steps must not straddle experts: the units per expert must
            // be a multiple of the narrowest lane group (4)
            if ((p.moe.I / 64) % 4 == 0 && p.moe.I % 64 == 0) return launch_typed<Q80x2, MODE>(p, s, grid_out);
            if ((p.moe.I / 32) % 4 == 0) return launch_typed<Q80x1, MODE>(p, s, grid_out);
            return hipErrorInvalidValue;
        }
        if ((p.K / 32) % 2 == 0) return launch_typed<Q80x2, MODE>(p, s, grid_out);
        return launch_typed<Q80x1, MODE>(p, s, grid_out);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qmv
