// The row-streaming matvec kernel shared by the single-token, fused-row,
// argmax and MoE expert entry points.
//
// Work split: a wave owns tiles of rows; inside a tile, groups of G lanes
// cooperate on one row (64/G rows side by side) and each lane also carries R
// independent row slots, so one step issues R x (64/G) rows of 128-bit loads.
// The activation vector x is staged once per workgroup in LDS together with
// its per-sub-block sums; every lane keeps the same unit position modulo G,
// so its 64 activations are read from LDS once per step and reused by all R
// rows.  The grid is persistent (exactly the resident workgroups) so the LDS
// staging is paid once per workgroup, not once per row.
//
// The per-row result is a fixed butterfly over the G lanes of fixed partial
// sums, so it depends only on (format, K, G, R) -- never on M, the grid or
// which rows share a tile.  That makes fused-row outputs and argmax values
// bit-identical to the plain matvec of the same rows.
//
// MoE modes (BebeLM page, section "核心算子": sigmoid router, top-k experts,
// bias used only to select, weights renormalised):
//  - kModeMoeGateUp: rows are the I row pairs (gate row j, up row j) of the
//    k selected experts, stacked; a tile holds 64/G gate rows in row slot 0
//    and the matching up rows, I further on in the expert's matrix, in slot
//    1, and the owner lane writes g, u and h = silu(g) * u.  Every workgroup
//    first derives the selection from the router logits (so no host round
//    trip and no extra launch), workgroup 0 publishes it.  Tiles never
//    straddle experts, so the expert of a tile is uniform.
//  - kModeMoeDown: row i is the concatenation over the k selected experts of
//    their down-projection row i, and x is the concatenation of w_s * h_s;
//    one row sum is then the weighted expert mixture, formed in a fixed
//    order.  G divides the units per expert, so the expert of each unit step
//    is uniform too.
//
// kModeShortConv (BebeLM page, section "门控短卷积": B, C, x = split(in_proj(h),
// 3); Bx = B * x; causal depthwise conv of kernel size 3 with a 2-position
// state; y = C * conv): the matrix is in_proj, 3M rows; a tile holds 64/G
// channels' B, C and x rows in row slots 0, 1 and 2, so the owner lane of a
// channel forms Bx, the convolution with the channel's state and taps, and y,
// and shifts the state; the 3M row results are never written.
//
// kModeSiluUp (BebeLM page, section "核心算子": the gated FFN h = silu(g) * u;
// FlareLLM page, section "推理层面的深度优化": gate and up as one stack): the
// matrix is a stacked gate+up of 2M rows; a tile holds 64/G gate rows in row
// slot 0 and the matching up rows, M further on, in slot 1, so the owner lane
// of a row has both results and writes only h = silu(g) * u.
#pragma once

#include <stdint.h>

#include "qmv_formats.h"

namespace qmv {

constexpr int kMaxSegments = 8;
constexpr int kXcds = 8;  // XCDs of an MI355X, each with its own L2
constexpr int kMaxExperts = 64;

// Row counts are below 2^31 (checked on the host), so every row and tile
// index is 32-bit and wave-uniform bookkeeping stays in scalar registers.
struct SegTable {
    int32_t n;
    int32_t start[kMaxSegments + 1];  // prefix sums of the segment row counts
    float *y[kMaxSegments];
};

struct MoeArgs {
    const float *logits;    // [E] router logits (gate/up launch)
    const float *bias;      // [E] selection bias (gate/up launch)
    int32_t E, k;
    int32_t *topk_idx;      // [k] written by the gate/up launch, read by the down launch
    float *topk_w;          // [k]
    float *h;               // [k][I] silu(g) * u: written by the gate/up launch, read by the down launch
    int64_t mat_bytes;      // bytes of one expert matrix
    int32_t rows_per_mat;   // gate/up launch: 2I
    int32_t units_per_mat;  // down launch: I / unit weights
    int32_t I;
};

struct RowsParams {
    const uint8_t *W;
    int32_t M;
    int32_t K;
    int64_t row_bytes;
    const float *x;
    SegTable seg;
    uint64_t *partials;  // argmax mode: one packed (value, index) key per workgroup
    MoeArgs moe;
    const float *conv_w;  // kModeShortConv: taps [M][3]
    float *conv_state;    // kModeShortConv: state [M][2], updated in place
};

enum {
    kModeStore = 0,
    kModeArgmax = 1,
    kModeMoeGateUp = 2,
    kModeMoeDown = 3,
    kModeSiluUp = 4,
    kModeShortConv = 5
};

// Packed argmax key: larger value first, then lower index.
__device__ __forceinline__ uint64_t argmax_key(float v, int32_t idx) {
    v = v + 0.0f;  // -0 -> +0 so equal values compare equal
    return ((uint64_t)float_key(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}

// Items whose weight loads a wave keeps in flight (register sets in its ring).
constexpr int kPipeDepth = 2;

// Formats whose row kernel streams faster with the next item requested only
// once the current item's first load has returned (measured: Q8_0 in
// two-block units, 128000 x 4096 96.3 against 99.2 us, 28672 x 4096 22.4
// against 23.7 us).  wait_first makes the first-issued load's register an
// operand of an empty asm, so the compiler waits for that load there.
template <class F>
struct Throttle {
    static constexpr bool kOn = false;
    __device__ static void wait_first(const typename F::Regs &) {}
};
template <>
struct Throttle<Q80x2> {
    static constexpr bool kOn = true;
    __device__ static __forceinline__ void wait_first(const Q80x2::Regs &r) {
        asm volatile("" ::"v"(r.a.x));
    }
};
template <>
struct Throttle<Q80x1> {
    static constexpr bool kOn = true;
    __device__ static __forceinline__ void wait_first(const Q80x1::Regs &r) {
        asm volatile("" ::"v"(r.c));
    }
};

// Floats of the padded LDS copy of x.
template <class F>
__host__ __device__ constexpr int lds_x_floats(int K) {
    return K + (K / F::kPadEvery) * 4;
}

// Store four consecutive activations (x[i..i+3]) into the padded LDS copy and
// add their group sum: the kSumGroup/4 consecutive lanes that hold one group
// combine with DPP moves (VALU only, no LDS round trip), so the sums need no
// extra pass over LDS.  Every lane of the wave must call this.
template <class F>
__device__ __forceinline__ void put_x4(float *xs, float *sums, int i, bool valid, float4 v) {
    if (valid) *reinterpret_cast<float4 *>(xs + i + (i / F::kPadEvery) * 4) = v;
    if constexpr (F::kSumGroup > 0) {
        constexpr int kLanes = F::kSumGroup / 4;
        static_assert(kLanes == 4 || kLanes == 8, "sum groups of 16 or 32 activations");
        float sum = (v.x + v.y) + (v.z + v.w);
        sum += dpp_f32<kDppXor1>(sum);
        sum += dpp_f32<kDppXor2>(sum);
        if (kLanes == 8) sum += dpp_f32<kDppHalfMirror>(sum);
        if (valid && (threadIdx.x % kLanes) == 0) sums[i / F::kSumGroup] = sum;
    }
}

// Stage x[0..K) in LDS, plus the sums of its consecutive groups of
// F::kSumGroup values.  x is stored padded (4 floats after every
// F::kPadEvery) so that the lanes' 16-byte reads spread over the LDS banks.
// Each thread issues NB loads of 4 floats at a time; `pre` runs after the
// first NB are issued, so work that is independent of x (the first weight
// loads) overlaps their latency.  Loads complete in order, so any x load
// issued after `pre` would also wait for what `pre` requested: NB is chosen
// so that the first batch covers all of x whenever it fits in 16 loads per
// thread.  K is a multiple of 32 (K >= 32), so a lane group is either wholly
// inside [0, K) or wholly outside.
struct NoPre {
    __device__ void operator()() const {}
};
template <class F, int NB, class Pre>
__device__ __forceinline__ void stage_x_nb(const BufSrc &xv, int K, float *xs, float *sums,
                                           Pre &pre) {
    const int nt = blockDim.x;
    auto batch = [&](int base0, bool first) {
        const int base = base0 + (int)threadIdx.x * 4;
        float4 v[NB];
#pragma unroll
        for (int j = 0; j < NB; j++)
            v[j] = __builtin_bit_cast(float4, xv.ld16((uint32_t)(base + j * nt * 4) * 4u));
        if (first) pre();
#pragma unroll
        for (int j = 0; j < NB; j++) {
            const int i = base + j * nt * 4;
            put_x4<F>(xs, sums, i, i < K, v[j]);
        }
    };
    // the first batch is peeled (straight-line code, so the waits for its x
    // loads do not cover the loads `pre` issues after them); the loop over
    // the rest is uniform over the workgroup
    batch(0, true);
    for (int base0 = nt * 4 * NB; base0 < K; base0 += nt * 4 * NB) batch(base0, false);
}
template <class F, class Pre = NoPre>
__device__ __forceinline__ void stage_x(const float *__restrict__ x, int K, float *xs,
                                        float *sums, Pre pre = Pre()) {
    // unconditional loads through a view of x (past K they read zeros), so
    // no branch makes the compiler wait for them early
    const BufSrc xv(reinterpret_cast<const uint8_t *>(x), (uint64_t)K * 4);
    const int per_thread = (K + (int)blockDim.x * 4 - 1) / ((int)blockDim.x * 4);
    if (per_thread <= 2)
        stage_x_nb<F, 2>(xv, K, xs, sums, pre);
    else if (per_thread <= 4)
        stage_x_nb<F, 4>(xv, K, xs, sums, pre);
    else if (per_thread <= 8)
        stage_x_nb<F, 8>(xv, K, xs, sums, pre);
    else
        stage_x_nb<F, 16>(xv, K, xs, sums, pre);
    __syncthreads();
}

__device__ __forceinline__ float sigmoidf(float v) { return 1.0f / (1.0f + expf(-v)); }
// silu(v) = v / (1 + e^-v), with the quotient as v times the hardware
// reciprocal (1 ulp) instead of the IEEE division sequence: a dozen fewer
// VALU instructions per row, which the gated launches pay once per tile.
__device__ __forceinline__ float siluf(float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + expf(-v));
}

// MoE selection from the router logits, done by every wave (each writes the
// same values into the workgroup's LDS slots, so it can use them without a
// barrier): scores s_e = sigmoid(r_e); rank by s_e + b_e (ties to the lower
// expert); weights = selected s_e over their sum.  Each lane (one expert)
// counts the experts that outrank it, reading the others' keys with
// v_readlane, so the selection is one pass of compares with no LDS round
// trips.  Wave 0 of workgroup 0 also writes topk_idx / topk_w.
__device__ __forceinline__ void moe_select(const MoeArgs &m, int32_t *sel, float *wsel) {
    const int e = threadIdx.x & (kWave - 1);
    const bool publish = blockIdx.x == 0 && threadIdx.x < kWave;
    const float s = e < m.E ? sigmoidf(m.logits[e]) : 0.f;
    const float v = e < m.E ? s + m.bias[e] + 0.0f : -__builtin_inff();  // -0 -> +0
    int rank = 0;
#pragma unroll
    for (int j = 0; j < kMaxExperts; j++) {
        const float vj = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), j));
        rank += (vj > v || (vj == v && j < e)) ? 1 : 0;
    }
    const bool chosen = e < m.E && rank < m.k;
    // sum of the selected scores (fixed order: DPP tree, total in lane 63)
    float ssum = group_sum<kWave>(chosen ? s : 0.f);
    ssum = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ssum), kWave - 1));
    if (chosen) {
        const float w = s / ssum;
        sel[rank] = e;
        wsel[rank] = w;
        if (publish) {
            m.topk_idx[rank] = e;
            m.topk_w[rank] = w;
        }
    }
}

// KS = 1: each wave owns whole tiles.  KS = 4: the four waves of a workgroup
// share each tile, wave w taking unit steps w, w + 4, ... (needs at least 4
// steps per row); their per-row partial sums meet in LDS and are added in
// wave order, so the result is still fixed by (format, K, G, KS).
// XR: a row is a single unit step, so every lane keeps the same unit for the
// whole launch and reads its activations from LDS once, after staging, into
// registers (modes whose x is one vector: not the MoE down launch).
// The body takes its workgroup index `bid` among `nblk` workgroups, so one
// launch can run two bodies side by side on separate workgroup ranges.
template <class F, int G, int R, int MODE, int KS, bool XR>
__device__ __forceinline__ void rows_body(const RowsParams &p, const int bid, const int nblk) {
    constexpr bool kMoe = MODE == kModeMoeGateUp || MODE == kModeMoeDown;
    extern __shared__ float smem[];
    float *xs = smem;
    float *sums = smem + lds_x_floats<F>(p.K);
    __shared__ int32_t sel[kMoe ? kMaxExperts : 1];
    __shared__ float wsel[kMoe ? kMaxExperts : 1];

    const int lane = threadIdx.x & (kWave - 1);
    // wave-uniform values are forced into scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int waves_per_block = blockDim.x / kWave;
    constexpr int P = kWave / G;  // rows side by side in one wave
    const int sub = lane / G, g = lane % G;
    const int U = p.K / F::kUnitWeights;
    const int iters = (U + G - 1) / G;  // unit steps per row
    // kModeSiluUp / kModeShortConv: the row slots are rows M apart in a
    // stack (gate and up; B, C and x); kModeMoeGateUp: I apart in an
    // expert's matrix (gate and up)
    constexpr bool kPair = MODE == kModeSiluUp || MODE == kModeShortConv || MODE == kModeMoeGateUp;
    static_assert(MODE != kModeSiluUp || R == 2, "gate and up slots");
    static_assert(MODE != kModeMoeGateUp || R == 2, "gate and up slots");
    static_assert(MODE != kModeShortConv || R == 3, "B, C and x slots");
    constexpr int kRowsPerTile = kPair ? P : R * P;
    const int ntiles = (p.M + kRowsPerTile - 1) / kRowsPerTile;
    const int tile_stride = KS == 1 ? nblk * waves_per_block : nblk;
    const int it0 = KS == 1 ? 0 : wave;  // this wave's first unit step of a tile
    static_assert(KS == 1 || KS == kBlockThreads / kWave, "K split over the workgroup's waves");
    // K-split partial sums: [tile parity][wave][row slot][row in wave]
    __shared__ float red[KS > 1 ? 2 * KS * R * P : 1];
    int tile_count = 0;
    const uint32_t rb = (uint32_t)p.row_bytes;

    // byte offset of row slot r inside a tile (rows of a tile are consecutive)
    uint32_t row_off[R];
#pragma unroll
    for (int r = 0; r < R; r++)
        row_off[r] = (uint32_t)(kPair ? r * (MODE == kModeMoeGateUp ? p.moe.I : p.M) + sub
                                      : r * P + sub) * rb;
    const uint32_t lane_uoff = F::unit_offset(g);

    float best_v = -__builtin_inff();
    int best_i = 0x7FFFFFFF;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; r++) acc[r] = 0.f;
    float xr[XR ? F::kUnitWeights : 1];  // XR: this lane's activations

    // The expert a unit step reads in the down launch (uniform: G divides the
    // units per expert, so a step never straddles two experts).
    auto step_slot = [&](int it) {
        return MODE == kModeMoeDown ? __builtin_amdgcn_readfirstlane((G * it) / p.moe.units_per_mat) : 0;
    };

    // One work item = (tile, unit step).  Items are software-pipelined: the
    // next item's weight loads are in flight while the current one is
    // multiplied, with two register sets used in turn (no copies, so no wait).
    // Tile bookkeeping is wave-uniform (scalar): each item reads through a
    // buffer view that starts at the tile's first row and ends at the end of
    // its matrix, so a lane only adds its own 32-bit offset, and rows past
    // the end (the ragged tail) or units past the last row's end read zeros
    // without touching memory.  Lanes whose unit lies past the row's end are
    // skipped by the multiply.
    auto issue = [&](typename F::Regs(&dst)[R], int t, int it) {
        t = __builtin_amdgcn_readfirstlane(t);
        it = __builtin_amdgcn_readfirstlane(it);
        int ustep = G * it;
        const int r0 = t * kRowsPerTile;
        const uint8_t *base;
        uint64_t avail;
        // A wave without items still issues its first loads (see the staging
        // below): past the end the view is empty and reads zeros.
        const bool live = r0 < p.M;
        if (MODE == kModeMoeGateUp) {
            // the tile's row pairs belong to one selected expert
            int slot = r0 / p.moe.I;
            slot = slot < p.moe.k ? slot : p.moe.k - 1;
            const int rin = r0 - slot * p.moe.I;
            const int ex = __builtin_amdgcn_readfirstlane(sel[slot]);  // uniform
            base = p.W + (int64_t)ex * p.moe.mat_bytes + (int64_t)rin * rb;
            avail = live ? (uint64_t)(p.moe.rows_per_mat - rin) * rb : 0;
        } else if (MODE == kModeMoeDown) {
            int slot = step_slot(it);
            slot = slot < p.moe.k ? slot : p.moe.k - 1;
            ustep -= slot * p.moe.units_per_mat;
            const int ex = __builtin_amdgcn_readfirstlane(sel[slot]);  // uniform
            base = p.W + (int64_t)ex * p.moe.mat_bytes + (int64_t)r0 * rb;
            avail = live ? (uint64_t)(p.M - r0) * rb : 0;
        } else {
            // stacked modes: the view runs to the end of the stack (R M rows)
            base = p.W + (int64_t)r0 * rb;
            avail = live ? (uint64_t)((kPair ? R * (int64_t)p.M : (int64_t)p.M) - r0) * rb : 0;
        }
        const BufSrc src(base, avail);
        // unit g + ustep: ustep is a multiple of 4, so the position inside a
        // block only depends on g
        const uint32_t uoff = lane_uoff + F::unit_offset(ustep);
#pragma unroll
        for (int r = 0; r < R; r++) dst[r] = F::load(src, row_off[r] + uoff, g);
    };
    auto finish_tile = [&](int t) {
        t = __builtin_amdgcn_readfirstlane(t);
        float tot[R];
#pragma unroll
        for (int r = 0; r < R; r++) {
            tot[r] = group_sum<G>(acc[r]);  // exact in the group's last lane
            acc[r] = 0.f;
        }
        bool owner = g == G - 1;
        if constexpr (KS > 1) {
            const int par = tile_count & 1;
            tile_count++;
            if (owner) {
#pragma unroll
                for (int r = 0; r < R; r++) red[((par * KS + wave) * R + r) * P + sub] = tot[r];
            }
            __syncthreads();
            owner = owner && wave == 0;
            if (owner) {
#pragma unroll
                for (int r = 0; r < R; r++) {
                    float v = red[((par * KS + 0) * R + r) * P + sub];
#pragma unroll
                    for (int w = 1; w < KS; w++) v += red[((par * KS + w) * R + r) * P + sub];
                    tot[r] = v;
                }
            }
        }
        const int r0 = t * kRowsPerTile;
        if constexpr (MODE == kModeMoeGateUp) {
            const int row = r0 + sub;  // row pair: slot * I + j
            if (owner && row < p.M) {
                const int slot = row / p.moe.I, j = row - slot * p.moe.I;
                float *gu = p.seg.y[0] + (int64_t)slot * 2 * p.moe.I;
                gu[j] = tot[0];
                gu[p.moe.I + j] = tot[1];
                p.moe.h[row] = siluf(tot[0]) * tot[1];
            }
        } else if constexpr (MODE == kModeSiluUp) {
            const int row = r0 + sub;
            if (owner && row < p.M) p.seg.y[0][row] = siluf(tot[0]) * tot[1];
        } else if constexpr (MODE == kModeShortConv) {
            const int ch = r0 + sub;
            if (owner && ch < p.M) {
                const float bx = tot[0] * tot[2];
                const float *w = p.conv_w + 3 * (int64_t)ch;
                float *st = p.conv_state + 2 * (int64_t)ch;
                const float s0 = st[0], s1 = st[1];
                // tap 2 takes the current input, tap 0 the oldest cached one
                const float conv = fmaf(w[2], bx, fmaf(w[1], s1, w[0] * s0));
                p.seg.y[0][ch] = tot[1] * conv;
                st[0] = s1;
                st[1] = bx;
            }
        } else if (MODE != kModeArgmax) {
            // segment of the tile's first row and the start of the next one:
            // compile-time indices over the table, all in scalar registers
            float *yb = p.seg.y[0];
            int sb = 0, next = INT32_MAX;
#pragma unroll
            for (int k = 1; k < kMaxSegments; k++) {
                if (k < p.seg.n) {
                    if (r0 >= p.seg.start[k]) {
                        sb = p.seg.start[k];
                        yb = p.seg.y[k];
                    } else if (next == INT32_MAX) {
                        next = p.seg.start[k];
                    }
                }
            }
            if (owner) {
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const int row = r0 + r * P + sub;
                    if (row >= p.M) continue;
                    if (row < next) {
                        yb[row - sb] = tot[r];
                    } else {  // the tile straddles a segment boundary
                        int s = 0;
                        while (s + 1 < p.seg.n && row >= p.seg.start[s + 1]) s++;
                        p.seg.y[s][row - p.seg.start[s]] = tot[r];
                    }
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < R; r++) {
                const int row = r0 + r * P + sub;
                const float v = tot[r] + 0.0f;
                if (owner && row < p.M && (v > best_v || (v == best_v && row < best_i))) {
                    best_v = v;
                    best_i = row;
                }
            }
        }
    };
    auto consume = [&](typename F::Regs(&src)[R], int t, int it) {
        t = __builtin_amdgcn_readfirstlane(t);
        it = __builtin_amdgcn_readfirstlane(it);
        const int u = g + G * it;
        // Lanes whose unit lies past the row's end compute on unit 0 (in
        // bounds of x and its sums) and keep their old sum: a select, not a
        // branch, so every path uses the set's registers and none leaves its
        // loads pending across the loop's back edge (with such a path the
        // compiler's waits before a refill also count the result stores
        // issued in between, and the ring ran one item deep).
        const bool valid = u < U;
        const int uc = valid ? u : 0;
        float part[R];
        if constexpr (XR) {
#pragma unroll
            for (int r = 0; r < R; r++) {
                part[r] = acc[r];
                F::dot(src[r], xr, sums, uc, part[r]);
            }
        } else {
            float xv[F::kUnitWeights];
            F::load_x(xs, uc, xv);
            // u indexes the (concatenated) x and its sums; the block-internal
            // position only depends on u mod 4, the same inside each expert
#pragma unroll
            for (int r = 0; r < R; r++) {
                part[r] = acc[r];
                F::dot(src[r], xv, sums, uc, part[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; r++) acc[r] = valid ? part[r] : acc[r];
        if (it + KS >= iters) finish_tile(t);  // this wave's last step of the tile
    };

    // Items of this wave: tiles t_first, t_first + stride, ..., each with
    // `iters` unit steps.  A round of tiles gives each wave one.  With many
    // rounds (long matrices) the wave's place in a round is chosen so that
    // the tiles covering one 128-byte line of y (kLineTiles consecutive
    // tiles) go to waves of one XCD (workgroup b runs on XCD b % 8): each
    // XCD then reads runs of consecutive rows and completes its lines of y
    // in its own L2, while the lines of a round still spread over all XCDs.
    // Measured (MI355X, cold): Q8_0 128000 x 4096 94.4 -> 90.7 us, 28672 x
    // 4096 22.5 -> 22.0 us, Q6_K 128000 x 4096 75.7 -> 73.2 us; with a few
    // rounds (the 4096 x 14336 and 28672 x 4096 Q4_K launches) it was
    // slower, so it applies from eight rounds on.  Any order of the tiles
    // gives the same results.
    constexpr int kLineTiles = kRowsPerTile >= 32 ? 1 : 32 / kRowsPerTile;
    int slot = KS == 1 ? bid * waves_per_block + wave : bid;
    if (KS == 1 && MODE != kModeArgmax && nblk % kXcds == 0 &&
        ntiles >= 8 * tile_stride && (nblk / kXcds * waves_per_block) % kLineTiles == 0) {
        const int j = (bid / kXcds) * waves_per_block + wave;  // place among the XCD's waves
        slot = ((j / kLineTiles) * kXcds + bid % kXcds) * kLineTiles + j % kLineTiles;
    }
    const int t_first = __builtin_amdgcn_readfirstlane(slot);
    const int my_tiles = t_first < ntiles ? (ntiles - 1 - t_first) / tile_stride + 1 : 0;
    const int steps = (iters - it0 + KS - 1) / KS;  // this wave's steps per tile
    const int n_items = my_tiles * steps;
    // ring of D register sets: D - 1 items' loads stay in flight while one
    // is multiplied
    constexpr int D = kPipeDepth;
    typename F::Regs buf[D][R];
    int ring_t[D], ring_it[D];  // the item each set holds (wave-uniform)
    ring_t[0] = t_first;
    ring_it[0] = it0;
    auto& bufA = buf[0];
    int &tA = ring_t[0], &itA = ring_it[0];

    if (MODE == kModeMoeGateUp) {
        // After the first activation loads are issued, each wave selects the
        // experts itself and requests its first weights; the activation
        // stores then wait only for x (loads complete in order).
        stage_x<F>(p.x, p.K, xs, sums, [&]() {
            moe_select(p.moe, sel, wsel);
            issue(bufA, tA, itA);
        });
        if constexpr (XR) F::load_x(xs, g < U ? g : 0, xr);
    } else if (MODE == kModeMoeDown) {
        if ((int)threadIdx.x < p.moe.k) {
            sel[threadIdx.x] = p.moe.topk_idx[threadIdx.x];
            wsel[threadIdx.x] = p.moe.topk_w[threadIdx.x];
        }
        __syncthreads();
        // x[s*I + j] = w_s * h_s[j], h written by the gate/up launch.
        // K = k*I is a multiple of 32, so sum groups never straddle slots.
        // The first pass's h values are loaded before the first weights are
        // requested, as in stage_x.
        const int I = p.moe.I, K = p.K;
        const int nt = blockDim.x;
        const BufSrc hv(reinterpret_cast<const uint8_t *>(p.moe.h), (uint64_t)K * 4);
        // kNB passes of 4 values per thread at a time: all their loads are
        // issued before any is used, so the batch pays one load latency
        constexpr int kNB = 4;
        auto batch = [&](int base0, bool first) {
            float4 hh[kNB];
            int base[kNB], sl[kNB];
#pragma unroll
            for (int i = 0; i < kNB; i++) {
                base[i] = base0 + i * nt * 4 + (int)threadIdx.x * 4;
                sl[i] = base[i] < K ? base[i] / I : 0;
                hh[i] = __builtin_bit_cast(float4, hv.ld16((uint32_t)(base[i] < K ? base[i] : 0) * 4u));
            }
            if (first) {
                issue(bufA, tA, itA);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = 0; i < kNB; i++) {
                const float w = wsel[sl[i]];
                put_x4<F>(xs, sums, base[i], base[i] < K,
                          make_float4(w * hh[i].x, w * hh[i].y, w * hh[i].z, w * hh[i].w));
            }
        };
        batch(0, true);
        for (int base0 = nt * 4 * kNB; base0 < K; base0 += nt * 4 * kNB) batch(base0, false);
        __syncthreads();
    } else {
        // the first item's weights are requested right after the first
        // activation loads: the two latencies overlap, and since loads
        // complete in order, the staging waits only for x, not for the
        // (slower) weights.  The issue is unconditional so that the wait
        // count for x is known at compile time.
        stage_x<F>(p.x, p.K, xs, sums, [&]() { issue(bufA, tA, itA); });
        if constexpr (XR) F::load_x(xs, g < U ? g : 0, xr);
    }

    // Every issue is unconditional, so the compiler's wait counters never
    // have to merge "maybe issued" states and each consume waits only for its
    // own loads.  Item q + 1 follows item q: the next unit step of the tile,
    // or the first step of the wave's next tile.  Past the wave's last item
    // the next tile lies past the last one, whose rows start at or after M:
    // those issues read through an empty view (zeros, no memory traffic).
    int t_last = t_first, it_last = it0;  // the newest issued item
    auto next_item = [&]() {
        if ((it_last += KS) >= iters) {
            it_last = it0;
            t_last += tile_stride;
        }
    };
#pragma unroll
    for (int j = 1; j < D - 1; j++) {
        next_item();
        ring_t[j] = t_last;
        ring_it[j] = it_last;
        issue(buf[j], t_last, it_last);
    }
    // Whole rounds of D items, each consume unconditional: no path around
    // the loop's back edge skips a consume, so no register set's loads can
    // still be pending when it is refilled.  (With a skippable consume the
    // compiler has to assume they might be, and with a result store between
    // the two sets' loads its wait before each refill then also waited for
    // the newest set's first load: the ring ran one item deep in the modes
    // that store.)
    int k = 0;
    for (; k + D <= n_items; k += D) {
#pragma unroll
        for (int j = 0; j < D; j++) {
            const int jn = (j + D - 1) % D;  // the set consumed one step ago
            next_item();
            ring_t[jn] = t_last;
            ring_it[jn] = it_last;
            // formats whose loads stream better with fewer in flight request
            // the next item only once the current one's first load is back
            if constexpr (Throttle<F>::kOn) Throttle<F>::wait_first(buf[j][0]);
            issue(buf[jn], t_last, it_last);
            // keep the multiply below the refill: hoisted above it, its
            // waits would hold the next loads back
            __builtin_amdgcn_sched_barrier(0);
            consume(buf[j], ring_t[j], ring_it[j]);
        }
    }
    // the last n_items - k (< D) items are already in flight in sets 0..
#pragma unroll
    for (int j = 0; j < D - 1; j++)
        if (k + j < n_items) consume(buf[j], ring_t[j], ring_it[j]);

    if (MODE == kModeArgmax) {
        __shared__ uint64_t wave_best[kMaxBlockThreads / kWave];
        uint64_t key = best_i < p.M ? argmax_key(best_v, best_i) : 0ull;
        for (int o = kWave / 2; o > 0; o >>= 1) {
            const uint64_t other = __shfl_xor(key, o, kWave);
            key = other > key ? other : key;
        }
        if (lane == 0) wave_best[wave] = key;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint64_t k = wave_best[0];
            for (int w = 1; w < waves_per_block; w++) k = wave_best[w] > k ? wave_best[w] : k;
            p.partials[bid] = k;
        }
    }
}

template <class F, int G, int R, int MODE, int KS, bool XR, int BT = kBlockThreads>
__global__ __launch_bounds__(BT) void rows_kernel(RowsParams p) {
    rows_body<F, G, R, MODE, KS, XR>(p, (int)blockIdx.x, (int)gridDim.x);
}

// Two row stacks of different formats sharing x in one launch (the fused
// rows of a mixed-format model, e.g. Q4_K Q and K with a Q6_K V): workgroups
// [0, g1) run the first stack's body, the rest the second's.  Each stack's
// rows are computed exactly as by its own launch (same lane group G).
template <class F1, class F2, int G, bool XR>
__global__ __launch_bounds__(kBlockThreads) void rows2_kernel(RowsParams p1, RowsParams p2, int g1) {
    if ((int)blockIdx.x < g1)
        rows_body<F1, G, 2, kModeStore, 1, XR>(p1, (int)blockIdx.x, g1);
    else
        rows_body<F2, G, 2, kModeStore, 1, XR>(p2, (int)blockIdx.x - g1, (int)gridDim.x - g1);
}

}  // namespace qmv
