// Prefill-size product Y = X W^T for many tokens on the matrix cores, and
// the ordered reduce of K-split partial sums shared with the verify
// product.  Exactness plan and weight policies: qmv_mfma.h.
#include "qmv_mfma.h"

namespace qmv {

namespace {

// Y[t][i] = sum over slices of the partial sums, in slice order.  The loads
// of up to eight slices are issued together before they are added, so the
// latency is paid once per eight slices, not once per slice.
__global__ __launch_bounds__(256) void gemm_n_reduce(const float *partial, int slices, int64_t nm,
                                                     float *Y) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= nm) return;
    float s = 0.f;
    for (int s0 = 0; s0 < slices; s0 += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = s0 + j < slices ? partial[(int64_t)(s0 + j) * nm + idx] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; j++)
            if (s0 + j < slices) s = (s0 + j == 0) ? v[j] : s + v[j];
    }
    Y[idx] = s;
}

// ---------------------------------------------------------------------------
// Prefill-size product (n up to thousands of tokens; BebeLM page, section
// "性能表现": prompts are processed in batches).  With many tokens there is
// parallelism across token blocks, so K is split only when rows and token
// blocks alone give too few workgroups: a workgroup owns 128 * RT rows, a
// block of 16 * TT tokens and a slice of consecutive 256-weight windows (all
// of K unless split).  A first kernel splits X once per call into the
// staged layout (bf16 hi/lo operand fragments and per-sub-block sums of
// every token block and window) in the workspace.  Per window the main
// kernel copies its token block's staged X into LDS, then multiplies while
// the next window's weights are in flight in a second register set.  Each
// weight sub-block's codes and scales are formed once and used by the TT
// token tiles.  Two workgroups share a compute unit, so one's X copy
// overlaps the other's multiply.  Every output is one fixed-order sum over
// the windows, or over the slices' partial sums added in slice order by a
// third kernel, so results are deterministic.
// Workgroups are mapped so that those sharing rows run on the same XCD
// (workgroups go to XCDs round-robin): their weights come from that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;

// TT: token tiles of 16 per workgroup (4; 2 or 1 when n is at most 32 or 16)
template <class F, int TT>
struct PfLayout {
    static constexpr int kPfTokens = 16 * TT;
    static constexpr int kVals = F::kNSub * 4 * kPfTokens * F::kKpl;  // = 256 * kPfTokens
    static constexpr int kBytes = kVals * 2 * 2 + F::kNSub * kPfTokens * 4;
    static_assert(kBytes % 16 == 0, "whole 16-byte chunks");
};

// Bytes of staged activations per (token block, window), the most any
// format takes (16 sub-blocks of sums), so the workspace size does not
// depend on the format.
constexpr size_t pf_window_bytes_max(int tt) { return (size_t)tt * 16 * (256 * 4 + 16 * 4); }

// X staging of one window for kPfTokens tokens; lane-group order as in the
// small-batch staging (tokens fastest within 16, then the four lane groups),
// then token tiles, then sub-blocks.
template <class F, int TT>
struct XStagePf {
    static constexpr int kPfTiles = TT, kPfTokens = 16 * TT;
    static constexpr int kGroups = kPfTokens * kWin / F::kKpl;
    static constexpr int kIters = kGroups / kThreads;
    static_assert(kGroups % kThreads == 0, "whole iterations");
    float v[kIters][F::kKpl];

    __device__ static __forceinline__ void coords(int it, int &j, int &q, int &t) {
        const int gi = (int)threadIdx.x + kThreads * it;
        const int tl = gi % 16;
        q = (gi / 16) % 4;
        const int tt = (gi / 64) % kPfTiles;
        j = gi / (64 * kPfTiles);
        t = tt * 16 + tl;
    }
    __device__ __forceinline__ void load(const BufSrc &xv, int K, int tok0, int win) {
#pragma unroll
        for (int it = 0; it < kIters; it++) {
            int j, q, t;
            coords(it, j, q, t);
            const int k = win * kWin + j * F::kSub + q * F::kKpl;
            const uint32_t off = ((uint32_t)(tok0 + t) * (uint32_t)K + (uint32_t)k) * 4u;
#pragma unroll
            for (int e = 0; e < F::kKpl / 4; e++) {
                const uint4 a = xv.ld16(off + 16 * e);
                v[it][4 * e] = __builtin_bit_cast(float, a.x);
                v[it][4 * e + 1] = __builtin_bit_cast(float, a.y);
                v[it][4 * e + 2] = __builtin_bit_cast(float, a.z);
                v[it][4 * e + 3] = __builtin_bit_cast(float, a.w);
            }
        }
    }
    __device__ __forceinline__ void store(uint8_t *base, int win, int K) const {
        using L = PfLayout<F, TT>;
#pragma unroll
        for (int it = 0; it < kIters; it++) {
            int j, q, t;
            coords(it, j, q, t);
            const int k = win * kWin + j * F::kSub + q * F::kKpl;
            const bool in_k = k < K;
            uint32_t hi[F::kKpl / 2], lo[F::kKpl / 2];
            float sum = 0.f;
#pragma unroll
            for (int i2 = 0; i2 < F::kKpl / 2; i2++) {
                f32x2 xx;
                xx.x = in_k ? v[it][F::perm(2 * i2)] : 0.f;
                xx.y = in_k ? v[it][F::perm(2 * i2 + 1)] : 0.f;
                const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(xx, bf16x2));
                const float h0 = __builtin_bit_cast(float, hb << 16);
                const float h1 = __builtin_bit_cast(float, hb & 0xFFFF0000u);
                f32x2 rr;
                rr.x = xx.x - h0;
                rr.y = xx.y - h1;
                const uint32_t lb = __builtin_bit_cast(uint32_t, __builtin_convertvector(rr, bf16x2));
                hi[i2] = hb;
                lo[i2] = lb;
                sum += (h0 + __builtin_bit_cast(float, lb << 16)) +
                       (h1 + __builtin_bit_cast(float, lb & 0xFFFF0000u));
            }
            const int pos = ((j * 4 + q) * kPfTokens + t) * F::kKpl;
            *reinterpret_cast<BFrag<F> *>(base + 2 * pos) = __builtin_bit_cast(BFrag<F>, hi);
            *reinterpret_cast<BFrag<F> *>(base + 2 * (L::kVals + pos)) = __builtin_bit_cast(BFrag<F>, lo);
            // lane groups q = 0..3 of (j, t) are the four 16-lane rows
            sum = rows_sum(sum);
            if (q == 0) reinterpret_cast<float *>(base + 4 * L::kVals)[j * kPfTokens + t] = sum;
        }
    }
};

// The staged activations of one (token block, window), written once per
// call: every row group's workgroups copy them into LDS instead of each
// loading and splitting X again.
template <class F, int TT>
__global__ __launch_bounds__(kThreads) void gemm_pf_prep(GemmParams p) {
    using L = PfLayout<F, TT>;
    const int tb = (int)blockIdx.x / p.windows, wi = (int)blockIdx.x % p.windows;
    const BufSrc xview(reinterpret_cast<const uint8_t *>(p.X), (uint64_t)p.n * (uint32_t)p.K * 4u);
    XStagePf<F, TT> xs;
    xs.load(xview, p.K, tb * 16 * TT, wi);
    xs.store(p.xprep + ((int64_t)tb * p.windows + wi) * L::kBytes, wi, p.K);
}

// RT 16-row tiles per wave (a workgroup owns 128 * RT rows): each X
// fragment read from LDS feeds RT row tiles' MFMAs, and the staged X of a
// window is shared by 128 * RT rows.
template <class F, int TT, int RT>
__global__ __launch_bounds__(kThreads, 4) void gemm_pf_kernel(GemmParams p, int token_blocks,
                                                            int wps) {
    using L = PfLayout<F, TT>;
    constexpr int kPfTiles = TT, kPfTokens = 16 * TT;
    constexpr int kRows = kRowsPerWG * RT;  // rows per workgroup
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int r = lane & 15, q = lane >> 4;
    // XCD-aware order: workgroups b and b + 8 share an XCD; consecutive
    // workgroups of one XCD take the (token block, K slice) pairs of one row
    // group
    const int b = (int)blockIdx.x;
    const int local = b / kXcds;
    const int cols = token_blocks * p.slices;
    const int cb = local % cols;
    const int tb = cb % token_blocks, slice = cb / token_blocks;
    const int rg = (b % kXcds) + kXcds * (local / cols);
    if (rg * kRows >= p.M) return;  // padding of the row groups
    const int row0 = __builtin_amdgcn_readfirstlane(rg * kRows + wave * 16 * RT);
    const int tok0 = tb * kPfTokens;
    const int nblocks = p.K / 32;
    // this workgroup's windows [w0, wtotal)
    const int w0 = slice * wps;
    const int wtotal = min((p.K + kWin - 1) / kWin, w0 + wps);

    const int rows_left = p.M - row0 > 0 ? p.M - row0 : 0;
    const BufSrc src(p.W + (int64_t)row0 * p.row_bytes,
                     (uint64_t)rows_left * (uint64_t)(uint32_t)p.row_bytes);

    auto nvalid_of = [&](int wi) {
        if constexpr (std::is_same<F, GQ80>::value) {
            const int left = nblocks - wi * 8;
            return left < 8 ? left : 8;
        } else {
            return F::kNSub;
        }
    };
    using Set = typename F::Regs[RT];
    auto wload = [&](Set &dst, int wi) {
        wi = __builtin_amdgcn_readfirstlane(wi < wtotal ? wi : wtotal - 1);
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
            dst[rt] = F::load(src, (uint32_t)(rt * 16 + r) * (uint32_t)p.row_bytes +
                                       (uint32_t)wi * F::kWinBytes,
                              q, nvalid_of(wi));
    };

    const uint32_t kmask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
    uint32_t kbias;
    asm("v_mov_b32 %0, %1" : "=v"(kbias) : "i"(kB16));
    f32x4 acc[RT][kPfTiles];
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int tt = 0; tt < kPfTiles; tt++) acc[rt][tt] = {0.f, 0.f, 0.f, 0.f};

    Set wcur;
    wload(wcur, w0);

    auto multiply = [&](const Set &w, const uint8_t *base, int wi) {
        const __bf16 *xhi = reinterpret_cast<const __bf16 *>(base);
        const __bf16 *xlo = xhi + L::kVals;
        const float *xsum = reinterpret_cast<const float *>(base + 4 * L::kVals);
        const int nsub = nvalid_of(wi);
        if constexpr (F::kCorr) {
#pragma unroll
            for (int j0 = 0; j0 < F::kNSub; j0 += 4)
#pragma unroll
                for (int tt = 0; tt < kPfTiles; tt++)
#pragma unroll
                    for (int rt = 0; rt < RT; rt++)
                        acc[rt][tt] = corr_mfma<F>(w[rt], xsum, kPfTokens, tt * 16, j0, r, q,
                                                   acc[rt][tt]);
        }
        // operand fragments of tile tt of sub-block j; each tile's are read
        // one tile ahead, so their LDS latency overlaps the previous tile's
        // MFMAs
        auto frag = [&](const __bf16 *x, int j, int tt) {
            const int fo = ((j * 4 + q) * kPfTokens + tt * 16 + r) * F::kKpl;
            return *reinterpret_cast<const Frag<F> *>(x + fo);
        };
        Frag<F> ah = frag(xhi, 0, 0), al = frag(xlo, 0, 0);
#pragma unroll
        for (int j = 0; j < F::kNSub; j++) {
            if (j >= nsub) break;
            Frag<F> bcode[RT];
            float scale[RT];
#pragma unroll
            for (int rt = 0; rt < RT; rt++) {
                bcode[rt] = F::codes(w[rt], j, kmask, kbias);
                scale[rt] = F::scale_of(w[rt], j);
            }
#pragma unroll
            for (int tt = 0; tt < kPfTiles; tt++) {
                // the next tile (past the last sub-block: none)
                const int jn = tt + 1 < kPfTiles ? j : j + 1;
                const int tn = tt + 1 < kPfTiles ? tt + 1 : 0;
                Frag<F> ahn = ah, aln = al;
                if (jn < F::kNSub) {
                    ahn = frag(xhi, jn, tn);
                    aln = frag(xlo, jn, tn);
                }
#pragma unroll
                for (int rt = 0; rt < RT; rt++) {
                    f32x4 c = {0.f, 0.f, 0.f, 0.f};
                    c = mfma<F>(ah, bcode[rt], c);
                    c = mfma<F>(al, bcode[rt], c);
                    acc[rt][tt][0] = fmaf(scale[rt], c[0], acc[rt][tt][0]);
                    acc[rt][tt][1] = fmaf(scale[rt], c[1], acc[rt][tt][1]);
                    acc[rt][tt][2] = fmaf(scale[rt], c[2], acc[rt][tt][2]);
                    acc[rt][tt][3] = fmaf(scale[rt], c[3], acc[rt][tt][3]);
                    // the sums are formed here: sunk to the next use of acc
                    // they would hold every tile's MFMA result at once
                    asm volatile("" : "+v"(acc[rt][tt]));
                }
                ah = ahn;
                al = aln;
                // keep each tile's operand reads and epilogue next to its
                // MFMAs (hoisting or sinking them across tiles would need
                // more registers than a wave has)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // Per window: stage X for the workgroup's tokens, then multiply while the
    // next window's weights are in flight (the load is unconditional: after
    // the last window it repeats it and nothing reads the result).  The X
    // load latency is hidden by the other workgroup on the compute unit (two
    // fit: one LDS buffer each).  The register sets trade places by a copy,
    // so the loop body exists once.
    for (int wi = w0; wi < wtotal; wi++) {
        const int wn = wi + 1 < wtotal ? wi + 1 : wi;
        {
            // the window's staged activations, copied by direct-to-LDS
            // 16-byte loads: each wave instruction fills 1 KB of LDS and no
            // register holds the data
            constexpr int kChunks = L::kBytes / 16;
            const uint8_t *g = p.xprep + ((int64_t)tb * p.windows + wi) * L::kBytes;
            for (int base = wave * kWave; base < kChunks; base += kThreads) {  // wave-uniform
                const int c = base + lane;
                if (c < kChunks)
                    __builtin_amdgcn_global_load_lds(
                        (const __attribute__((address_space(1))) void *)(g + 16 * (int64_t)c),
                        (__attribute__((address_space(3))) void *)(smem + 16 * base), 16, 0, 0);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();
        Set wnext;
        wload(wnext, wn);
        multiply(wcur, smem, wi);
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < RT; rt++) wcur[rt] = wnext[rt];
    }

    float *out = p.slices == 1 ? p.Y : p.partial + (int64_t)slice * p.n * p.M;
    // The output offsets only depend on the launch: formed here, after the
    // loop (the empty asm keeps the compiler from computing them up front
    // and holding them in registers through the multiply loop).
    int row_l = row0 + r, tok_l = tok0 + 4 * q;
    asm volatile("" : "+v"(row_l), "+v"(tok_l));
#pragma unroll
    for (int rt = 0; rt < RT; rt++) {
        const int row = row_l + rt * 16;
        if (row < p.M) {
            float *yr = out + row;
#pragma unroll
            for (int tt = 0; tt < kPfTiles; tt++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int t = tok_l + tt * 16 + i;
                    if (t < p.n) yr[(int64_t)t * p.M] = acc[rt][tt][i];
                }
        }
    }
}

template <class F, int TT, int RT>
hipError_t launch_pf_tt(GemmParams p, const PfPlan &plan, hipStream_t s) {
    const size_t lds = (size_t)PfLayout<F, TT>::kBytes;
    hipError_t e = ensure_lds((const void *)gemm_pf_kernel<F, TT, RT>, lds);
    if (e != hipSuccess) return e;
    p.slices = plan.slices;
    const int64_t grid = (int64_t)plan.rg_pad * plan.token_blocks * plan.slices;
    const int64_t prep_grid = (int64_t)plan.token_blocks * p.windows;
    if (grid > 0x7FFFFFFFll || prep_grid > 0x7FFFFFFFll) return hipErrorInvalidValue;
    e = launch_aux(gemm_pf_prep<F, TT>, dim3((unsigned)prep_grid), dim3(kThreads), 0, s, p);
    if (e != hipSuccess) return e;
    e = launch_main(gemm_pf_kernel<F, TT, RT>, dim3((unsigned)grid), dim3(kThreads), lds, s, p,
                    plan.token_blocks, plan.wps);
    if (e != hipSuccess || plan.slices == 1) return e;
    const int64_t nm = (int64_t)p.n * p.M;
    return launch_aux(gemm_n_reduce, dim3((unsigned)((nm + 255) / 256)), dim3(256), 0, s,
                      (const float *)p.partial, p.slices, nm, p.Y);
}

// formats whose two-tile waves fit the register budget of two workgroups
// per compute unit
template <class F>
constexpr bool two_tiles() {
    return std::is_same<F, GQ4K>::value || std::is_same<F, GQ5K>::value;
}

template <class F>
hipError_t launch_pf(GemmParams p, hipStream_t s) {
    PfPlan plan = pf_plan(p.M, p.K, p.n);
    if (plan.rt == 2) {
        if constexpr (two_tiles<F>()) return launch_pf_tt<F, 4, 2>(p, plan, s);
        // the same plan with one-tile waves: twice the workgroups, same slices
        plan.rt = 1;
        plan.rg_pad = (int)(((p.M + kRowsPerWG - 1) / kRowsPerWG + kXcds - 1) / kXcds * kXcds);
    }
    switch (plan.tt) {
    case 4: return launch_pf_tt<F, 4, 1>(p, plan, s);
    case 2: return launch_pf_tt<F, 2, 1>(p, plan, s);
    default: return launch_pf_tt<F, 1, 1>(p, plan, s);
    }
}

}  // namespace

// Prefill launch plan.  Tokens per workgroup: 64 (TT = 4) when n fills
// them, else 32 or 16.  Enough workgroups means 384 (1.5 per compute unit
// of a 256-CU part; two fit).  In order of preference:
//  1. two row tiles per wave (256-row workgroups, 64 tokens), no K split;
//  2. two row tiles and K split into the fewest slices (powers of two up to
//     16) that give enough workgroups, if each slice keeps at least twelve
//     256-weight windows;
//  3. one row tile per wave (128 rows), no split;
//  4. one row tile and the fewest slices (at least two windows each) that
//     give enough, or the most there can be.
// Splitting K beat taking fewer tokens per workgroup, and long slices paid
// for the two-tile waves' shared X reads (us per call, old plan of fewer
// tokens -> this one; the 4096 x 14336 down projection at n = 64 / 256 /
// 512: 51 -> 38, 130 -> 93, 193 -> 163, and at n = 1024 one tile without a
// split 329 against two tiles with two slices 311; the 4096 x 4096 one at
// n = 256 / 512: 42 -> 38, 62 -> 59).  Short slices did not pay for two
// tiles (4096 x 4096 at n = 512 with four slices of four windows: 62.6
// against 58.8 us; at n = 1024 with two of eight: 102.9 against 97.0), and
// a split did not pay where there were enough workgroups (gate+up 28672 x
// 4096 at n = 256: 149 us, 169 with two slices).  The plan depends only on
// (M, K, n), so the workspace size does too.
PfPlan pf_plan(int64_t M, int64_t K, int64_t n) {
    constexpr int64_t kEnough = 384;
    constexpr int kLongSlice = 12;
    const int wtotal = (int)((K + kWin - 1) / kWin);
    const int tt = n > 32 ? 4 : n > 16 ? 2 : 1;
    const int tb = (int)((n + 16 * tt - 1) / (16 * tt));
    auto groups = [&](int rows) {
        const int64_t g = (M + rows - 1) / rows;
        return (int)((g + kXcds - 1) / kXcds * kXcds);
    };
    const int rg2 = groups(2 * kRowsPerWG), rg1 = groups(kRowsPerWG);
    PfPlan pl{};
    pl.tt = tt;
    pl.token_blocks = tb;
    auto with = [&](int rt, int rg) {
        pl.rt = rt;
        pl.rg_pad = rg;
        return pl;
    };
    // the fewest slices that give g workgroups enough (or the most allowed)
    auto split = [&](int64_t g) {
        pl.slices = 1;
        pl.wps = wtotal;
        if (g >= kEnough) return true;
        for (int ks = 2; ks <= 16 && wtotal / ks >= 2; ks *= 2) {
            pl.wps = (wtotal + ks - 1) / ks;
            pl.slices = (wtotal + pl.wps - 1) / pl.wps;  // no empty slice
            if (g * pl.slices >= kEnough) return true;
        }
        return false;
    };
    if (tt == 4 && split((int64_t)rg2 * tb) && (pl.slices == 1 || pl.wps >= kLongSlice))
        return with(2, rg2);
    split((int64_t)rg1 * tb);
    return with(1, rg1);
}

// Workspace: the slices' partial sums (split K only), then the staged
// activations of every (token block, window), 256-byte aligned.
static size_t pf_partial_bytes(const PfPlan &pl, int64_t M, int64_t n) {
    const size_t b = pl.slices > 1 ? (size_t)pl.slices * (size_t)n * (size_t)M * sizeof(float) : 0;
    return (b + 255) / 256 * 256;
}

size_t gemm_workspace(int64_t M, int64_t K, int64_t n) {
    const PfPlan pl = pf_plan(M, K, n);
    const size_t windows = (size_t)((K + kWin - 1) / kWin);
    return pf_partial_bytes(pl, M, n) + (size_t)pl.token_blocks * windows * pf_window_bytes_max(pl.tt);
}

hipError_t launch_gemm(int type, const uint8_t *W, int64_t M, int64_t K, int64_t n, const float *X,
                       float *Y, void *ws, hipStream_t s) {
    GemmParams p{};
    p.W = W;
    p.M = (int32_t)M;
    p.K = (int32_t)K;
    p.n = (int32_t)n;
    p.row_bytes = (int32_t)row_bytes_of(type, K);
    p.X = X;
    p.Y = Y;
    p.partial = reinterpret_cast<float *>(ws);
    p.windows = (int32_t)((K + kWin - 1) / kWin);
    p.xprep = reinterpret_cast<uint8_t *>(ws) + pf_partial_bytes(pf_plan(M, K, n), M, n);
    switch (type) {
    case kQ4K: return launch_pf<GQ4K>(p, s);
    case kQ5K: return launch_pf<GQ5K>(p, s);
    case kQ6K: return launch_pf<GQ6K>(p, s);
    case kQ80: return launch_pf<GQ80>(p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_slice_reduce(const float *partial, int slices, int64_t nm, float *Y,
                               hipStream_t s) {
    return launch_aux(gemm_n_reduce, dim3((unsigned)((nm + 255) / 256)), dim3(256), 0, s, partial,
                      slices, nm, Y);
}

}  // namespace qmv
