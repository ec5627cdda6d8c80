// Small-batch verify: Y[n][M] = X[n][K] . dequant(W)^T for n <= 16 on the
// matrix cores (FlareLLM page, section "推理层面的深度优化": n-gram speculative
// decoding checks several drafted tokens against the same weights).
// Arithmetic (exact integer codes, X as bf16 hi + lo, f32 scales): qmv_mfma.h.
//
// Work split.  A 512-thread workgroup (one per compute unit) owns a K slice
// -- all of K unless K is long -- and walks groups of 16-row tiles.  Its
// eight waves split each group: `ks` waves share a tile along K (wave kw takes
// the slice's windows kw, kw + ks, ...) and 8 / ks tiles are in work at once.
// Each wave builds the X fragments of its windows once (coalesced loads,
// through a per-wave LDS staging area into registers), streams its share of
// the tiles' weights with the next tiles' loads in flight (16-byte loads per
// lane, rearranged across the lane groups by row swaps: qmv_mfma.h), and
// leaves each tile's 16 x 16 partial product in LDS;
// after every kBatch tiles the workgroup adds the ks partials of each tile in
// wave order and writes the outputs.  So a K slice needs no workspace and no
// second launch.  Only K longer than one slice (more than 4096 weights: two
// windows of 256 per wave, the most whose X fragments and weight sets fit the
// registers without spills) splits into slices whose partial sums go to the
// workspace and are added in slice order by a second kernel.  Every output is
// a fixed-order sum, so results are deterministic.
//
// n <= 8 packs both halves of X into one MFMA operand: A rows 0-7 hold the
// tokens' bf16 hi parts and rows 8-15 their lo parts, so one MFMA per
// sub-block covers both (C rows t and t + 8 are added in the reduction) and
// the X fragments take half the registers.  For 8 < n <= 16, A holds the 16
// tokens' hi parts and a second MFMA their lo parts.
#include "qmv_mfma.h"

namespace qmv {

namespace {

struct VerifyParams {
    const uint8_t *W;
    int32_t M, K, n;
    int32_t row_bytes;
    const float *X;
    float *out;         // Y [n][M], or the [slices][n][M] partial sums
    int32_t slices;     // K slices
    int32_t wps;        // windows (256 weights) per slice
    int32_t ks;         // waves sharing a tile along K (1, 2, 4 or 8)
    int32_t groups;     // tile groups of 8 / ks tiles
    int32_t per_slice;  // workgroups per slice
};

constexpr int kBatch = 4;  // tiles per wave between two reductions

// WPW: windows per wave (registers for their X fragments); PACK: n <= 8 with
// hi and lo in one operand; D: register sets in the weight ring (D - 1 tiles
// in flight while one is multiplied).
template <class F, int WPW, bool PACK, int D>
__global__ __launch_bounds__(kThreads, 1) void verify_kernel(VerifyParams p) {
    constexpr int kWaves = kThreads / kWave;
    // per-wave 16 x 16 partial products [token][row], double-buffered by batch
    __shared__ float red[2][kBatch][kWaves][kTok * 16];
    // per-wave staging of activations: 8 tokens x one window (64 chunks of
    // 16 bytes), chunk m of token t stored at m ^ t
    __shared__ uint4 xst[kWaves][8 * (kWin / 4)];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int r = lane & 15, q = lane >> 4;
    const int ks = p.ks, rs = kWaves / ks;
    const int kw = wave % ks, rg = wave / ks;
    const int slice = (int)blockIdx.x % p.slices;
    const int gfirst = (int)blockIdx.x / p.slices;
    const int wtotal = (p.K + kWin - 1) / kWin;
    const int ws0 = slice * p.wps;
    const int ws1 = min(wtotal, ws0 + p.wps);
    const int nblocks = p.K / 32;  // Q8_0 blocks per row (last window)
    const int n_items =
        gfirst < p.groups ? (p.groups - 1 - gfirst) / p.per_slice + 1 : 0;  // uniform
    const uint32_t lane_off = (uint32_t)r * (uint32_t)p.row_bytes;

    auto win_of = [&](int i) { return ws0 + kw + ks * i; };
    auto nvalid_of = [&](int wi) {
        if constexpr (std::is_same<F, GQ80>::value) {
            const int left = nblocks - wi * 8;
            return left < 8 ? left : 8;
        } else {
            return F::kNSub;
        }
    };

    // ---- weights of one item (this wave's tile of a group, its windows) ----
    // Tiles past the last row and windows past the slice read through an
    // empty view: zeros, no memory traffic.
    auto load_item = [&](typename F::Wide(&wr)[WPW], int k) {
        const int g = gfirst + p.per_slice * k;
        const int row0 = __builtin_amdgcn_readfirstlane((g * rs + rg) * 16);
        const int rows_left = p.M - row0 > 0 ? p.M - row0 : 0;
        const uint8_t *base = p.W + (int64_t)(rows_left > 0 ? row0 : 0) * p.row_bytes;
#pragma unroll
        for (int i = 0; i < WPW; i++) {
            int wi = win_of(i);
            const bool valid = wi < ws1;
            wi = __builtin_amdgcn_readfirstlane(valid ? wi : ws0);
            const BufSrc src(base, valid ? (uint64_t)rows_left * (uint32_t)p.row_bytes : 0);
            wr[i] = F::fetch(src, lane_off + (uint32_t)wi * F::kWinBytes, q, nvalid_of(wi));
        }
    };

    // ---- X fragments of this wave's windows, in registers for the launch ----
    Frag<F> xa[WPW][F::kNSub];                                  // hi (PACK: hi / lo rows)
    Frag<F> xb[PACK ? 1 : WPW][PACK ? 1 : F::kNSub];           // lo (8 < n <= 16)
    float xc[WPW][F::kNSub / 4];                                // -(hi + lo) sums, corr operand
    const int tok = PACK ? (r & 7) : r;
    const bool lo_row = PACK && r >= 8;
    const BufSrc xview(reinterpret_cast<const uint8_t *>(p.X), (uint64_t)p.n * (uint32_t)p.K * 4u);

    // Every lane splits half of a window's sub-blocks per pass.  Packed X
    // (one pass): the two lanes of a token (operand rows r and r + 8) take
    // the first and the second half and swap what the other needs with one
    // DPP move per dword (row_ror:8 exchanges lanes r and r + 8).  16 tokens
    // (two passes): pass h covers sub-blocks h * kNSub / 2 .. for all lanes.
    constexpr int kOwn = F::kNSub / 2;
    constexpr int kPasses = PACK ? 1 : 2;
    auto own_j = [&](int jj, int h) {
        return jj + (PACK ? (lo_row ? F::kNSub / 2 : 0) : h * (F::kNSub / 2));
    };
    auto partner = [](uint32_t v) {  // every lane has a source: no fill value needed
        return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kDppRowRor8, 0xF, 0xF, false);
    };

    // Activations reach the operand layout through LDS.  One pass stages
    // 8 KB per wave: 8 tokens x 256 values (packed) or 16 tokens x the pass's
    // 128 values, read with each load instruction covering whole token runs
    // (lane l: 16-byte chunk l % kChunks of token l / kChunks of the pair),
    // then each lane reads back its own token's k-slots.  Chunk m of staged
    // token t sits at m ^ (t % 8), so the writes and the operand-order reads
    // (eight tokens at one chunk) fall in distinct banks.  Tokens past n
    // read as zero (past the end of the view).
    constexpr int kChunks = PACK ? kWin / 4 : kWin / 8;  // 16-byte chunks per staged token
    auto x_issue = [&](int i, int h, uint4(&g)[8]) {
        const int t_lane = lane / kChunks, c = lane % kChunks;
        const uint32_t base = ((uint32_t)t_lane * (uint32_t)p.K + (uint32_t)win_of(i) * kWin) * 4u +
                              (uint32_t)(h * kChunks + c) * 16u;
#pragma unroll
        for (int u = 0; u < 8; u++)
            g[u] = xview.ld16(base + (uint32_t)(u * (kWave / kChunks)) * (uint32_t)p.K * 4u);
    };
    auto x_stage = [&](int h, const uint4(&g)[8], float(&v)[kOwn][F::kKpl]) {
        uint4 *st = xst[wave];
        const int t_lane = lane / kChunks, c = lane % kChunks;
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int t = u * (kWave / kChunks) + t_lane;
            st[t * kChunks + (c ^ (t & 7))] = g[u];
        }
        // a wave's LDS accesses complete in order: the reads below see the
        // writes above, and the next pass's writes follow these reads
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int jj = 0; jj < kOwn; jj++) {
            const int m0 = (own_j(jj, h) * F::kSub + q * F::kKpl) / 4 - h * kChunks;
#pragma unroll
            for (int e = 0; e < F::kKpl / 4; e++) {
                const uint4 a = st[tok * kChunks + ((m0 + e) ^ (tok & 7))];
                v[jj][4 * e] = __builtin_bit_cast(float, a.x);
                v[jj][4 * e + 1] = __builtin_bit_cast(float, a.y);
                v[jj][4 * e + 2] = __builtin_bit_cast(float, a.z);
                v[jj][4 * e + 3] = __builtin_bit_cast(float, a.w);
            }
        }
        __builtin_amdgcn_wave_barrier();
    };
    // bf16 hi + lo split into the operand layout (slots 2i, 2i+1 hold values
    // perm(2i), perm(2i+1)), and the sub-block sums of hi + lo for the
    // correction MFMA (two bf16 pair dots with (1, 1) per value pair).  Only
    // Q8_0 windows run past K (32-weight blocks): those activations count as
    // zero.  Windows past the slice are converted but never multiplied.
    const bf16x2 ones2 = __builtin_bit_cast(bf16x2, 0x3F803F80u);
    auto x_convert = [&](int i, int h, const float (&v)[kOwn][F::kKpl]) {
        const int wi = win_of(i);
        float sums[F::kNSub];
#pragma unroll
        for (int jj = 0; jj < kOwn; jj++) {
            bool in = true;
            if constexpr (std::is_same<F, GQ80>::value)
                in = wi * kWin + own_j(jj, h) * F::kSub + q * F::kKpl < p.K;
            uint32_t hi[F::kKpl / 2], lo[F::kKpl / 2];
            float sum = 0.f;
#pragma unroll
            for (int i2 = 0; i2 < F::kKpl / 2; i2++) {
                f32x2 xx;
                xx.x = in ? v[jj][F::perm(2 * i2)] : 0.f;
                xx.y = in ? v[jj][F::perm(2 * i2 + 1)] : 0.f;
                const bf16x2 hv = __builtin_convertvector(xx, bf16x2);
                const uint32_t hb = __builtin_bit_cast(uint32_t, hv);
                f32x2 rr;
                rr.x = xx.x - __builtin_bit_cast(float, hb << 16);
                rr.y = xx.y - __builtin_bit_cast(float, hb & 0xFFFF0000u);
                const bf16x2 lv = __builtin_convertvector(rr, bf16x2);
                hi[i2] = hb;
                lo[i2] = __builtin_bit_cast(uint32_t, lv);
                sum = __builtin_amdgcn_fdot2_f32_bf16(hv, ones2, sum, false);
                sum = __builtin_amdgcn_fdot2_f32_bf16(lv, ones2, sum, false);
            }
            // lane groups q = 0..3 of (token, j) are the four 16-lane rows
            sum = rows_sum(sum);
            if constexpr (PACK) {
                // keep the half this lane's operand row holds, send the other
                uint32_t keep[F::kKpl / 2], recv[F::kKpl / 2];
#pragma unroll
                for (int i2 = 0; i2 < F::kKpl / 2; i2++) {
                    keep[i2] = lo_row ? lo[i2] : hi[i2];
                    recv[i2] = partner(lo_row ? hi[i2] : lo[i2]);
                }
                const float srecv = __builtin_bit_cast(float, partner(__builtin_bit_cast(uint32_t, sum)));
                uint32_t first[F::kKpl / 2], second[F::kKpl / 2];
#pragma unroll
                for (int i2 = 0; i2 < F::kKpl / 2; i2++) {
                    first[i2] = lo_row ? recv[i2] : keep[i2];
                    second[i2] = lo_row ? keep[i2] : recv[i2];
                }
                xa[i][jj] = __builtin_bit_cast(Frag<F>, first);
                xa[i][jj + F::kNSub / 2] = __builtin_bit_cast(Frag<F>, second);
                sums[jj] = lo_row ? srecv : sum;
                sums[jj + F::kNSub / 2] = lo_row ? sum : srecv;
            } else {
                const int j = jj + h * kOwn;
                xa[i][j] = __builtin_bit_cast(Frag<F>, hi);
                xb[i][j] = __builtin_bit_cast(Frag<F>, lo);
                sums[j] = sum;
            }
        }
        // corr operand of sub-blocks j0 .. j0+3: lane (r, q) gives token r's
        // sum of sub-block j0 + q (PACK: the lo rows add nothing)
        const int jlo = PACK ? 0 : h * kOwn, jhi = PACK ? F::kNSub : (h + 1) * kOwn;
#pragma unroll
        for (int j0 = 0; j0 < F::kNSub; j0 += 4) {
            if (j0 < jlo || j0 >= jhi) continue;
            const float s = q == 0 ? sums[j0] : q == 1 ? sums[j0 + 1] : q == 2 ? sums[j0 + 2] : sums[j0 + 3];
            xc[i][j0 / 4] = lo_row ? 0.f : -s;
        }
    };

    // The activations are requested first, then the first items' weights, so
    // the two latencies overlap and the conversion waits only for what is in
    // flight then (loads complete in order).
    typename F::Wide ring[D][WPW];
    {
        // packed X: both windows in flight before the weights; otherwise the
        // first window's first pass
        uint4 g0[8], g1[8];
        float v[kOwn][F::kKpl];
        x_issue(0, 0, g0);
        if constexpr (WPW > 1 && PACK) x_issue(1, 0, g1);
        // every wave's activation loads go ahead of all weight loads in the
        // compute unit's memory pipeline
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int j = 0; j < D - 1; j++) load_item(ring[j], j);
#pragma unroll
        for (int i = 0; i < WPW; i++) {
#pragma unroll
            for (int h = 0; h < kPasses; h++) {
                if constexpr (PACK) {
                    x_stage(h, i == 0 ? g0 : g1, v);
                } else {
                    if (i + h > 0) x_issue(i, h, g0);
                    x_stage(h, g0, v);
                }
                x_convert(i, h, v);
            }
        }
    }

    const uint32_t kmask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
    uint32_t kbias;
    asm("v_mov_b32 %0, %1" : "=v"(kbias) : "i"(kB16));

    // ---- this wave's partial product of one tile over its windows ----
    auto multiply = [&](const typename F::Wide(&ww)[WPW]) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < WPW; i++) {
            const int wi = win_of(i);
            if (wi >= ws1) break;  // wave-uniform: every lane stays active
            // one window's unpacked registers at a time
            __builtin_amdgcn_sched_barrier(0);
            const typename F::Regs wr = F::regs(ww[i]);
            const int nsub = nvalid_of(wi);
            if constexpr (F::kCorr) {
#pragma unroll
                for (int j0 = 0; j0 < F::kNSub; j0 += 4)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xc[i][j0 / 4], F::corr_q(wr, j0, q),
                                                               acc, 0, 0, 0);
            }
            // four sub-blocks at a time: their MFMA chains are independent, so
            // they issue back to back and their results are consumed together
#pragma unroll
            for (int jb = 0; jb < F::kNSub; jb += 4) {
                if (jb >= nsub) break;
                Frag<F> bq[4];
                float scale[4];
                f32x4 c[4];
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    bq[t] = F::codes(wr, jb + t, kmask, kbias);
                    scale[t] = jb + t < nsub ? F::scale_of(wr, jb + t) : 0.f;
                }
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    c[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                    c[t] = mfma<F>(xa[i][jb + t], bq[t], c[t]);
                    if constexpr (!PACK) c[t] = mfma<F>(xb[i][jb + t], bq[t], c[t]);
                }
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    acc[0] = fmaf(scale[t], c[t][0], acc[0]);
                    acc[1] = fmaf(scale[t], c[t][1], acc[1]);
                    acc[2] = fmaf(scale[t], c[t][2], acc[2]);
                    acc[3] = fmaf(scale[t], c[t][3], acc[3]);
                }
            }
        }
        return acc;
    };

    // ---- the ks partials of each tile of a batch, added in wave order ----
    float *out = p.out + (p.slices > 1 ? (int64_t)slice * p.n * p.M : 0);
    auto reduce = [&](int buf, int nslots, int kfirst) {
        __syncthreads();
        const int per_tile = p.n * 16;
        const int total = nslots * rs * per_tile;
        for (int o = (int)threadIdx.x; o < total; o += kThreads) {
            const int s = o / (rs * per_tile);
            const int rem = o - s * (rs * per_tile);
            const int rgo = rem / per_tile;
            const int e = rem - rgo * per_tile;
            const int t = e >> 4, rr = e & 15;
            const int g = gfirst + p.per_slice * (kfirst + s);
            const int row = (g * rs + rgo) * 16 + rr;
            float v = 0.f;
            for (int k = 0; k < ks; k++) {
                const float *w = red[buf][s][k + ks * rgo];
                v += w[t * 16 + rr];
                if constexpr (PACK) v += w[(t + 8) * 16 + rr];
            }
            if (row < p.M) out[(int64_t)t * p.M + row] = v;
        }
    };

    // Items in a ring of D register sets: the set multiplied one step ago
    // receives the item D - 1 ahead (past the last item: empty views).
    int batch = 0, slot = 0;
    for (int k0 = 0; k0 < n_items; k0 += D) {
#pragma unroll
        for (int j = 0; j < D; j++) {
            const int k = k0 + j;
            load_item(ring[(j + D - 1) % D], k + D - 1);
            if (k < n_items) {
                const f32x4 acc = multiply(ring[j]);
                float *w = red[batch & 1][slot][wave];
#pragma unroll
                for (int e = 0; e < 4; e++) w[(4 * q + e) * 16 + r] = acc[e];
                slot++;
                if (slot == kBatch || k == n_items - 1) {
                    reduce(batch & 1, slot, k - slot + 1);
                    batch++;
                    slot = 0;
                }
            }
        }
    }
}

// Launch plan: K slices of at most 8 * (most windows per wave) windows, the
// most waves per tile along K (a power of two, at most the slice's windows),
// and enough windows per wave to cover the slice.
struct VerifyPlan {
    bool pack;
    int wpw, slices, wps, ks, groups;
};

VerifyPlan verify_plan(int64_t M, int64_t K, int32_t n) {
    VerifyPlan pl{};
    pl.pack = n <= 8;
    // four windows per wave (packed X) spilled registers in every format
    const int max_wpw = 2;
    const int W = (int)((K + kWin - 1) / kWin);
    const int cap = (kThreads / kWave) * max_wpw;
    pl.slices = (W + cap - 1) / cap;
    pl.wps = (W + pl.slices - 1) / pl.slices;
    pl.slices = (W + pl.wps - 1) / pl.wps;  // no empty slice
    pl.ks = kThreads / kWave;
    while (pl.ks > 1 && pl.ks > pl.wps) pl.ks >>= 1;
    const int need = (pl.wps + pl.ks - 1) / pl.ks;
    pl.wpw = need <= 1 ? 1 : 2;
    const int rs = (kThreads / kWave) / pl.ks;
    const int64_t tiles = (M + 15) / 16;
    pl.groups = (int)((tiles + rs - 1) / rs);
    return pl;
}

// Ring depth: three register sets where the X fragments leave room (packed
// X: 32 registers per window), else two.
template <class F, int WPW, bool PACK>
constexpr int ring_depth() {
    return PACK ? 3 : 2;
}

template <class F, int WPW, bool PACK>
hipError_t launch_verify_kernel(VerifyParams p, hipStream_t s) {
    constexpr int D = ring_depth<F, WPW, PACK>();
    const auto k = verify_kernel<F, WPW, PACK, D>;
    const int64_t grid = (int64_t)p.per_slice * p.slices;
    return launch_main(k, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
}

template <class F>
hipError_t launch_verify_typed(VerifyParams p, const VerifyPlan &pl, hipStream_t s) {
    if (pl.pack) {
        if (pl.wpw == 2) return launch_verify_kernel<F, 2, true>(p, s);
        return launch_verify_kernel<F, 1, true>(p, s);
    }
    if (pl.wpw == 2) return launch_verify_kernel<F, 2, false>(p, s);
    return launch_verify_kernel<F, 1, false>(p, s);
}

}  // namespace

size_t gemm_n_workspace(int64_t M, int64_t K, int32_t n) {
    const int64_t slices = verify_plan(M, K, n).slices;
    return slices > 1 ? (size_t)slices * (size_t)n * (size_t)M * sizeof(float) : 0;
}

hipError_t launch_gemm_n(int type, const uint8_t *W, int64_t M, int64_t K, int32_t n,
                         const float *X, float *Y, void *ws, hipStream_t s) {
    const VerifyPlan pl = verify_plan(M, K, n);
    VerifyParams p{};
    p.W = W;
    p.M = (int32_t)M;
    p.K = (int32_t)K;
    p.n = n;
    p.row_bytes = (int32_t)row_bytes_of(type, K);
    p.X = X;
    p.out = pl.slices > 1 ? reinterpret_cast<float *>(ws) : Y;
    p.slices = pl.slices;
    p.wps = pl.wps;
    p.ks = pl.ks;
    p.groups = pl.groups;
    // one workgroup per compute unit, shared evenly by the slices
    int per_slice = device_cu_count() / pl.slices;
    if (per_slice > pl.groups) per_slice = pl.groups;
    if (per_slice < 1) per_slice = 1;
    p.per_slice = per_slice;
    hipError_t e;
    switch (type) {
    case kQ4K: e = launch_verify_typed<GQ4K>(p, pl, s); break;
    case kQ5K: e = launch_verify_typed<GQ5K>(p, pl, s); break;
    case kQ6K: e = launch_verify_typed<GQ6K>(p, pl, s); break;
    case kQ80: e = launch_verify_typed<GQ80>(p, pl, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || pl.slices == 1) return e;
    return launch_slice_reduce(p.out, pl.slices, (int64_t)n * M, Y, s);
}

}  // namespace qmv
