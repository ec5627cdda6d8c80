// Small-batch verify: Y[n][M] = X[n][K] . dequant(W)^T for n <= 16 on the
// matrix cores (FlareLLM page, section "推理层面的深度优化": n-gram speculative
// decoding checks several drafted tokens against the same weights).
//
// Exactness plan (the result stays within the f32 matvec's 1e-5 sum|w x|):
//  - the MFMA's weight operand holds the raw integer codes, which bf16
//    represents exactly (written 0x43uu = 128 + u); the f32 scale d*sc is
//    applied to the f32 MFMA result once per sub-block, and the per-sub-block
//    correction (the +128 and the min) times the activation sums is itself a
//    small product, sums[token][j] x corr[j][row], done by one f32 MFMA
//    (16x16x4) per four sub-blocks straight into the accumulator;
//  - X is split into bf16 hi + lo (two MFMAs into one accumulator), so the
//    only representation error is |x - hi - lo| <= 2^-18 |x|.
// Operand roles: tokens are the MFMA M side (A = X fragment), weight rows the
// N side (B = codes), so a lane's accumulators all belong to the row whose
// block header that lane loaded and the scales apply lane-locally.
//   v_mfma_f32_16x16x32_bf16 (Q4_K, Q8_0: one 32-weight sub-block / block) and
//   v_mfma_f32_16x16x16_bf16 (Q6_K: one 16-weight sub-block); lane l of wave
//   supplies A[l%16][kpl*(l/16) + t], B[kpl*(l/16) + t][l%16] and holds
//   C[4*(l/16) + i][l%16].
//
// Work split: K is cut into slices of KW windows of 256 weights (KW = 1 or
// 2, chosen so that there are enough (128-row group, slice) pairs).  An
// 8-wave workgroup, one per compute unit, is bound to one slice: it stages X
// for the slice once in LDS (bf16 hi/lo in the MFMA operand layout plus
// per-sub-block sums), each wave reads its part of the X fragments into
// registers once, then streams 16-row tiles (one MFMA tile) of the slice,
// the next tile's weights in flight while the current one is multiplied.  With more than one slice, each writes its partial sums to
// the workspace and a second kernel adds them in slice order
// (deterministic, no atomics).
#include "qmv_device.h"
#include "qmv_internal.h"

#include <type_traits>

namespace qmv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTok = 16;                 // MFMA M side: tokens, n padded to 16
constexpr int kWin = 256;                // weights per window (one super-block)
constexpr uint32_t kB16 = 0x43004300u;  // bf16 128.0 in both halves

struct GemmParams {
    const uint8_t *W;
    int32_t M, K, n;
    int32_t row_bytes;
    const float *X;
    float *Y;          // final output (one slice) ...
    float *partial;    // ... or [slices][n][M] partial sums
    int32_t row_groups;
    int32_t slices;
};

constexpr int kThreads = 512;  // 8 waves
constexpr int kRowsPerWG = 128;

// ---------------------------------------------------------------------------
// Format policies.  kSub: weights per MFMA sub-block (= MFMA K); kNSub:
// sub-blocks per 256-weight window; kKpl: operand values per lane.
// slot(i): where weight i (0..255) of a window sits in the operand layout, as
// (sub-block j, lane group q, slot t).  load(src, off, q, nvalid): the bytes
// lane group q needs from the window starting `off` bytes into the view.
// ---------------------------------------------------------------------------
struct GQ4K {
    static constexpr int kSub = 32, kNSub = 8, kKpl = 8, kWinBytes = 144;
    struct Regs {
        uint4 hdr;
        uint2 piece[4];  // nibble bytes 32c + 8q .. +8, c = 0..3
    };
    // k-slot t of lane group q in sub-block 2c + h is nibble h of byte
    // 8q + pi(t) of chunk c, pi = (0 2 1 3 4 6 5 7): the order in which two
    // and-or operations pull nibble pairs out of a dword.
    __device__ static constexpr int perm(int b) { return (b & 4) | ((b & 1) << 1) | ((b & 2) >> 1); }
    __device__ static void slot(int i, int &j, int &q) {
        const int c = i / 64, h = (i % 64) / 32, l = i % 32;
        j = 2 * c + h;
        q = l / 8;
    }
    __device__ static Regs load(const BufSrc &src, uint32_t off, int q, int) {
        Regs r;
        r.hdr = src.ld16(off);
#pragma unroll
        for (int c = 0; c < 4; c++) r.piece[c] = src.ld8(off + 16 + 32 * c + 8 * q);
        return r;
    }
    // mask and bf16 bias arrive in registers, so each code dword is one
    // v_and_or_b32 (plus a shift): a VOP3 instruction takes no literal here
    __device__ static bf16x8 codes(const Regs &r, int j, uint32_t mask, uint32_t bias) {
        const uint2 p = r.piece[j >> 1];
        const int sh = (j & 1) * 4;
        uint32_t d[4];
        d[0] = ((p.x >> sh) & mask) | bias;
        d[1] = ((p.x >> (sh + 8)) & mask) | bias;
        d[2] = ((p.y >> sh) & mask) | bias;
        d[3] = ((p.y >> (sh + 8)) & mask) | bias;
        return __builtin_bit_cast(bf16x8, d);
    }
    // y += scale * C - corr * sum(x): w = d*sc*q - dmin*m and the codes are q + 128.
    // Scale bytes: sub-blocks 0-3 take the low 6 bits of bytes 4-7 (scale)
    // and 8-11 (min); 4-7 the low / high nibble of bytes 12-15 plus the top
    // two bits of bytes 4-7 / 8-11.
    static constexpr bool kCorr = true;
    __device__ static float scale_of(const Regs &r, int j) { return hdr_scale(r.hdr, j); }
    __device__ static float corr_of(const Regs &r, int j) { return hdr_corr(r.hdr, j); }
    __device__ static int hdr_sc(const uint4 &hdr, int j) {
        const int sh = 8 * (j & 3);
        return j < 4 ? (int)((hdr.y >> sh) & 63)
                     : (int)(((hdr.w >> sh) & 15) | ((((hdr.y >> sh) >> 6) & 3) << 4));
    }
    __device__ static int hdr_m(const uint4 &hdr, int j) {
        const int sh = 8 * (j & 3);
        return j < 4 ? (int)((hdr.z >> sh) & 63)
                     : (int)((((hdr.w >> sh) >> 4) & 15) | ((((hdr.z >> sh) >> 6) & 3) << 4));
    }
    __device__ static float hdr_scale(const uint4 &hdr, int j) {
        return half_bits_to_float(hdr.x) * (float)hdr_sc(hdr, j);
    }
    __device__ static float hdr_corr(const uint4 &hdr, int j) {
        const float dmin = half_bits_to_float(hdr.x >> 16);
        return fmaf(128.0f, hdr_scale(hdr, j), dmin * (float)hdr_m(hdr, j));
    }
};

// Q5_K (BebeLM page, section "局限与未来": Q5_K_M): the Q4_K super-block plus
// 32 bytes of fifth bits; bit 2c + h of high byte l is the fifth bit of
// weight 64c + 32h + l, i.e. bit j of byte l for sub-block j.  Lane group q
// takes high bytes 8q .. 8q + 8 (the same l as its nibble bytes), and each
// code dword gets its two fifth bits or-ed in at bit 4 of both halves, so
// the bf16 codes are 128 + q with q in 0..31 (exact).
struct GQ5K {
    static constexpr int kSub = 32, kNSub = 8, kKpl = 8, kWinBytes = 176;
    struct Regs {
        uint4 hdr;
        uint2 qh;        // high bytes 8q .. 8q + 8
        uint2 piece[4];  // nibble bytes 32c + 8q .. +8, c = 0..3
    };
    __device__ static constexpr int perm(int b) { return GQ4K::perm(b); }
    __device__ static void slot(int i, int &j, int &q) { GQ4K::slot(i, j, q); }
    __device__ static Regs load(const BufSrc &src, uint32_t off, int q, int) {
        Regs r;
        r.hdr = src.ld16(off);
        r.qh = src.ld8(off + 16 + 8 * q);
#pragma unroll
        for (int c = 0; c < 4; c++) r.piece[c] = src.ld8(off + 48 + 32 * c + 8 * q);
        return r;
    }
    __device__ static bf16x8 codes(const Regs &r, int j, uint32_t mask, uint32_t bias) {
        const uint2 p = r.piece[j >> 1];
        const int sh = (j & 1) * 4;
        uint32_t d[4];
        d[0] = ((p.x >> sh) & mask) | bias | (((r.qh.x >> j) & 0x00010001u) << 4);
        d[1] = ((p.x >> (sh + 8)) & mask) | bias | (((r.qh.x >> (j + 8)) & 0x00010001u) << 4);
        d[2] = ((p.y >> sh) & mask) | bias | (((r.qh.y >> j) & 0x00010001u) << 4);
        d[3] = ((p.y >> (sh + 8)) & mask) | bias | (((r.qh.y >> (j + 8)) & 0x00010001u) << 4);
        return __builtin_bit_cast(bf16x8, d);
    }
    static constexpr bool kCorr = true;
    __device__ static float scale_of(const Regs &r, int j) { return GQ4K::hdr_scale(r.hdr, j); }
    __device__ static float corr_of(const Regs &r, int j) { return GQ4K::hdr_corr(r.hdr, j); }
};

struct GQ6K {
    static constexpr int kSub = 16, kNSub = 16, kKpl = 4, kWinBytes = 210;
    struct Regs {
        uint32_t ql[2][2][2];  // [n][g&1][hh]: QL bytes 64n + 32(g&1) + 16hh + 4q .. +4
        uint32_t qh[2][2];     // [n][hh]: QH bytes 32n + 16hh + 4q .. +4
        uint4 sc;
        uint32_t d;
    };
    // weight i = 128n + 32g + 16hh + 4q + t, sub-block j = 8n + 2g + hh
    __device__ static constexpr int perm(int b) { return b; }
    __device__ static void slot(int i, int &j, int &q) {
        const int n = i / 128, g = (i % 128) / 32, l = i % 32, hh = l / 16;
        j = 8 * n + 2 * g + hh;
        q = (l % 16) / 4;
    }
    __device__ static Regs load(const BufSrc &src, uint32_t off, int q, int) {
        Regs r;
#pragma unroll
        for (int n = 0; n < 2; n++)
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int hh = 0; hh < 2; hh++)
                    r.ql[n][a][hh] = src.ld4(off + 64 * n + 32 * a + 16 * hh + 4 * q);
#pragma unroll
        for (int n = 0; n < 2; n++)
#pragma unroll
            for (int hh = 0; hh < 2; hh++) r.qh[n][hh] = src.ld4(off + 128 + 32 * n + 16 * hh + 4 * q);
        r.sc = src.ld16(off + 192);
        r.d = src.ld2(off + 208);
        return r;
    }
    __device__ static s16x4 codes(const Regs &r, int j, uint32_t, uint32_t) {
        const int n = j / 8, g = (j % 8) / 2, hh = j % 2;
        const uint32_t lo = (r.ql[n][g & 1][hh] >> (4 * (g >> 1))) & 0x0F0F0F0Fu;
        const uint32_t hi = ((r.qh[n][hh] >> (2 * g)) & 0x03030303u) << 4;
        const uint32_t u = lo | hi;  // four 6-bit codes, one per byte
        uint32_t d[2];
        d[0] = __builtin_amdgcn_perm(0x43434343u, u, 0x04010400u);  // [u0, 43, u1, 43]
        d[1] = __builtin_amdgcn_perm(0x43434343u, u, 0x04030402u);  // [u2, 43, u3, 43]
        return __builtin_bit_cast(s16x4, d);
    }
    // w = d*sc*(u - 32) and the codes are u + 128: y += d*sc*C - 160*d*sc*sum(x)
    static constexpr bool kCorr = true;
    __device__ static float scale_of(const Regs &r, int j) {
        const uint32_t w = j < 4 ? r.sc.x : j < 8 ? r.sc.y : j < 12 ? r.sc.z : r.sc.w;
        return half_bits_to_float(r.d) * (float)(int32_t)(int8_t)((w >> (8 * (j & 3))) & 0xFFu);
    }
    __device__ static float corr_of(const Regs &r, int j) { return 160.0f * scale_of(r, j); }
};

struct GQ80 {
    // a window is 8 consecutive Q8_0 blocks; block j is sub-block j
    static constexpr int kSub = 32, kNSub = 8, kKpl = 8, kWinBytes = 272;
    struct Regs {
        uint2 q[8];
        uint32_t d[8];
    };
    __device__ static constexpr int perm(int b) { return b; }
    __device__ static void slot(int i, int &j, int &q) {
        j = i / 32;
        q = (i % 32) / 8;
    }
    // nvalid of the window's 8 blocks exist (the rest repeat the last one)
    __device__ static Regs load(const BufSrc &src, uint32_t off, int q, int nvalid) {
        Regs r;
#pragma unroll
        for (int b = 0; b < 8; b++) {
            const uint32_t p = off + 34 * (b < nvalid ? b : nvalid - 1);
            r.d[b] = src.ld2(p);
            r.q[b] = src.ld8(p + 2 + 8 * q);
        }
        return r;
    }
    __device__ static bf16x8 codes(const Regs &r, int j, uint32_t, uint32_t) {
        const uint32_t w[2] = {r.q[j].x, r.q[j].y};
        uint32_t d[4];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            // signed byte -> f32 (exact) -> its upper 16 bits are the bf16
            const float f0 = sbyte<0>(w[h]), f1 = sbyte<1>(w[h]);
            const float f2 = sbyte<2>(w[h]), f3 = sbyte<3>(w[h]);
            d[2 * h] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1),
                                             __builtin_bit_cast(uint32_t, f0), 0x07060302u);
            d[2 * h + 1] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f3),
                                                 __builtin_bit_cast(uint32_t, f2), 0x07060302u);
        }
        return __builtin_bit_cast(bf16x8, d);
    }
    static constexpr bool kCorr = false;  // signed codes, no offset, no min
    __device__ static float scale_of(const Regs &r, int j) { return half_bits_to_float(r.d[j]); }
    __device__ static float corr_of(const Regs &, int) { return 0.f; }
};

template <class F>
using Frag = typename std::conditional<F::kKpl == 8, bf16x8, s16x4>::type;
template <class F>
using BFrag = typename std::conditional<F::kKpl == 8, bf16x8, bf16x4>::type;

// acc[token][row] -= sum over four sub-blocks of sums[token][j] * corr[j][row]:
// an f32 MFMA with K = 4, lane (r, q) supplying the sum of token r and the
// correction of its row for sub-block j0 + q.
template <class F, class Regs>
__device__ __forceinline__ f32x4 corr_mfma(const Regs &w, const float *sums, int stride, int tok,
                                           int j0, int r, int q, f32x4 acc) {
    const float a = -sums[(j0 + q) * stride + tok + r];
    const float b = F::corr_of(w, j0 + q);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

template <class F>
__device__ __forceinline__ f32x4 mfma(const Frag<F> &a, const Frag<F> &b, f32x4 c) {
    if constexpr (F::kKpl == 8)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// LDS per window buffer and part: hi and lo fragments [j][q][token][kKpl]
// bf16 (8 KB each), then the per-(j, token) sums of hi + lo.
template <class F>
struct WinLayout {
    static constexpr int kVals = F::kNSub * 4 * kTok * F::kKpl;  // = 16 * 256
    static constexpr int kBytes = kVals * 2 * 2 + F::kNSub * kTok * 4;
};

template <class F>
size_t gemm_lds_bytes(int KW) {
    return (size_t)KW * WinLayout<F>::kBytes;
}

// X staging for the KW windows of a slice, in two halves: load reads the f32
// activations into registers (unconditional loads through a view of
// X[0..n): tokens past n read zeros, so no branch waits for the data),
// store splits them into bf16 hi + lo, writes them in the operand layout and
// adds the per-sub-block sums.  A lane takes the kKpl consecutive
// activations of one (sub-block j, lane group q, token t), with t fastest:
// consecutive lanes write consecutive 16-byte operand slots (no LDS bank
// conflicts), and the four lane groups of a sub-block sit 16 lanes apart in
// one wave, so their sum is two lane exchanges.
template <class F, int KW>
struct XStage {
    static constexpr int kGroups = kTok * kWin / F::kKpl;  // per window
    static constexpr int kIters = KW * kGroups / kThreads;
    static_assert(KW * kGroups % kThreads == 0, "whole iterations");
    static_assert(F::kSub / F::kKpl == 4, "four lane groups per sub-block");
    float v[kIters][F::kKpl];

    __device__ static __forceinline__ void coords(int it, int &win, int &j, int &q, int &t) {
        const int gi = (int)threadIdx.x + kThreads * it;
        win = gi / kGroups;
        const int gg = gi % kGroups;
        t = gg % kTok;
        q = (gg / kTok) % 4;
        j = gg / (4 * kTok);
    }

    __device__ __forceinline__ void load(const GemmParams &p, const BufSrc &xv, int wfirst) {
#pragma unroll
        for (int it = 0; it < kIters; it++) {
            int win, j, q, t;
            coords(it, win, j, q, t);
            const int k = (wfirst + win) * kWin + j * F::kSub + q * F::kKpl;
            const uint32_t off = ((uint32_t)t * (uint32_t)p.K + (uint32_t)k) * 4u;
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

    // activations past K (the slice's or a last partial Q8_0 window) are zeroed
    __device__ __forceinline__ void store(uint8_t *smem, int wfirst, int K) const {
        using L = WinLayout<F>;
#pragma unroll
        for (int it = 0; it < kIters; it++) {
            int win, j, q, t;
            coords(it, win, j, q, t);
            const int k = (wfirst + win) * kWin + j * F::kSub + q * F::kKpl;
            const bool in_k = k < K;  // K is a multiple of the group size
            // operand slots (2i, 2i+1) hold activations (perm(2i), perm(2i+1)):
            // one packed conversion per slot pair for hi, one for lo
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
            uint8_t *base = smem + (size_t)win * L::kBytes;
            const int pos = ((j * 4 + q) * kTok + t) * F::kKpl;
            *reinterpret_cast<BFrag<F> *>(base + 2 * pos) = __builtin_bit_cast(BFrag<F>, hi);
            *reinterpret_cast<BFrag<F> *>(base + 2 * (L::kVals + pos)) = __builtin_bit_cast(BFrag<F>, lo);
            // lane groups q = 0..3 of (j, t) are lanes t, t + 16, t + 32, t + 48
            sum += __shfl_xor(sum, 16, kWave);
            sum += __shfl_xor(sum, 32, kWave);
            if (q == 0) reinterpret_cast<float *>(base + 4 * L::kVals)[j * kTok + t] = sum;
        }
    }
};

// A workgroup is bound to one K-slice: it stages X for the slice once, then
// each wave walks 16-row tiles of the matrix (tile_first, tile_first +
// stride, ...) with two register sets in turn, so the next tile's weights are
// in flight while the current one is multiplied.  Tiles past the last row
// read through an empty view (zeros, no memory traffic).
template <class F, int KW>
__global__ __launch_bounds__(kThreads) void gemm_n_kernel(GemmParams p, int wg_per_slice) {
    using L = WinLayout<F>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    constexpr int kWaves = kThreads / kWave;
    const int r = lane & 15, q = lane >> 4;
    const int slice = (int)blockIdx.x % p.slices, gidx = (int)blockIdx.x / p.slices;
    const int nblocks = p.K / 32;                // Q8_0 blocks per row (last window)
    const int wtotal = (p.K + kWin - 1) / kWin;  // windows in a row
    const int wfirst = slice * KW;
    const int row_tiles = (p.M + 15) / 16;
    const int stride = wg_per_slice * kWaves;
    const uint32_t lane_off = (uint32_t)r * (uint32_t)p.row_bytes;

    auto nvalid_of = [&](int wi) {
        if constexpr (std::is_same<F, GQ80>::value) {
            const int left = nblocks - wi * 8;
            return left < 8 ? left : 8;
        } else {
            return F::kNSub;
        }
    };
    // every window of the slice for one tile (windows past the row's end
    // repeat the last one and are skipped by the multiply)
    auto load_tile = [&](typename F::Regs(&wr)[KW], int tile) {
        const int row0 = __builtin_amdgcn_readfirstlane(tile * 16);
        const int rows_left = p.M - row0 > 0 ? p.M - row0 : 0;
        const BufSrc src(p.W + (int64_t)row0 * p.row_bytes,
                         (uint64_t)rows_left * (uint64_t)(uint32_t)p.row_bytes);
#pragma unroll
        for (int i = 0; i < KW; i++) {
            int wi = wfirst + i < wtotal ? wfirst + i : wtotal - 1;
            wi = __builtin_amdgcn_readfirstlane(wi);
            wr[i] = F::load(src, lane_off + (uint32_t)wi * F::kWinBytes, q, nvalid_of(wi));
        }
    };

    const int t0 = __builtin_amdgcn_readfirstlane(gidx * kWaves + wave);
    typename F::Regs bufA[KW], bufB[KW];
    load_tile(bufA, t0);
    {
        const BufSrc xview(reinterpret_cast<const uint8_t *>(p.X),
                           (uint64_t)p.n * (uint32_t)p.K * 4u);
        XStage<F, KW> xs;
        xs.load(p, xview, wfirst);
        xs.store(smem, wfirst, p.K);
    }
    __syncthreads();

    // The slice's X fragments and activation sums are the same for every row
    // tile, so each lane reads its part of them from LDS once, into registers
    // (64 VGPRs per window; one 8-wave workgroup per compute unit is two
    // waves per SIMD, which leaves room for them: 126-245 VGPRs, no spills),
    // and the tile loop does no LDS reads.  Gate+up 28672 x 4096 at n = 8, 16:
    // 27.6 / 30.0 -> 26.6 / 28.7 us per call.
    Frag<F> xh[KW][F::kNSub], xl[KW][F::kNSub];
    float xc[KW][F::kNSub / 4];
#pragma unroll
    for (int i = 0; i < KW; i++) {
        const uint8_t *base = smem + (size_t)i * L::kBytes;
        const __bf16 *xhi = reinterpret_cast<const __bf16 *>(base);
        const __bf16 *xlo = xhi + L::kVals;
        const float *xs = reinterpret_cast<const float *>(base + 4 * L::kVals);
#pragma unroll
        for (int j = 0; j < F::kNSub; j++) {
            const int fo = ((j * 4 + q) * kTok + r) * F::kKpl;
            xh[i][j] = *reinterpret_cast<const Frag<F> *>(xhi + fo);
            xl[i][j] = *reinterpret_cast<const Frag<F> *>(xlo + fo);
        }
#pragma unroll
        for (int j0 = 0; j0 < F::kNSub; j0 += 4) xc[i][j0 / 4] = -xs[(j0 + q) * kTok + r];
    }

    // code-packing constants in registers (one SGPR, one VGPR)
    const uint32_t kmask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
    uint32_t kbias;
    asm("v_mov_b32 %0, %1" : "=v"(kbias) : "i"(kB16));
    float *out = p.slices == 1 ? p.Y : p.partial + (int64_t)slice * p.n * p.M;

    auto multiply_store = [&](const typename F::Regs(&wr)[KW], int tile) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < KW; i++) {
            const int wi = wfirst + i;
            if (wi >= wtotal) break;
            const int nsub = nvalid_of(wi);
            if constexpr (F::kCorr) {
#pragma unroll
                for (int j0 = 0; j0 < F::kNSub; j0 += 4)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        xc[i][j0 / 4], F::corr_of(wr[i], j0 + q), acc, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < F::kNSub; j++) {
                if (j >= nsub) break;
                const Frag<F> &ah = xh[i][j], &al = xl[i][j];
                const Frag<F> b = F::codes(wr[i], j, kmask, kbias);
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
                c = mfma<F>(ah, b, c);
                c = mfma<F>(al, b, c);
                const float scale = F::scale_of(wr[i], j);
                acc[0] = fmaf(scale, c[0], acc[0]);
                acc[1] = fmaf(scale, c[1], acc[1]);
                acc[2] = fmaf(scale, c[2], acc[2]);
                acc[3] = fmaf(scale, c[3], acc[3]);
            }
        }
        // tokens 4q .. 4q+3 of this lane's row
        const int row = tile * 16 + r;
        if (row < p.M) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int t = 4 * q + i;
                if (t < p.n) out[(int64_t)t * p.M + row] = acc[i];
            }
        }
    };

    // two register sets in turn: the set just multiplied receives the tile
    // after next
    for (int t = t0; t < row_tiles; t += 2 * stride) {
        load_tile(bufB, t + stride);
        multiply_store(bufA, t);
        if (t + stride >= row_tiles) break;
        load_tile(bufA, t + 2 * stride);
        multiply_store(bufB, t + stride);
    }
}

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

// Windows per slice: 2 if that still gives 512 (128-row group, slice)
// pairs, two per compute unit of a 256-CU part, else 1 (measured against
// 256, 384 and 768 pairs: the 32-layer verify pass was 1-3% faster).  Four
// windows per slice would give fewer slices on large matrices, but their
// kernel needs 146-227 VGPRs against 64-126 for two: gate+up 28672 x 4096
// took 32.7-34.5 us with four and 27.5-31.5 us with two (n = 8, 16).  The
// plan depends only on M and K, so the workspace size does too.
int windows_per_slice(int64_t M, int64_t K) {
    const int64_t groups = (M + kRowsPerWG - 1) / kRowsPerWG;
    const int64_t wtotal = (K + kWin - 1) / kWin;
    return groups * ((wtotal + 1) / 2) >= 512 ? 2 : 1;
}

// One 8-wave workgroup per compute unit; each slice gets an equal share of
// the workgroups (at most one per 8 row tiles).
template <class F, int KW>
hipError_t launch_kw(GemmParams p, hipStream_t s) {
    const int wtotal = (p.K + kWin - 1) / kWin;
    p.row_groups = (p.M + kRowsPerWG - 1) / kRowsPerWG;
    p.slices = (wtotal + KW - 1) / KW;
    const size_t lds = gemm_lds_bytes<F>(KW);
    hipError_t e = ensure_lds((const void *)gemm_n_kernel<F, KW>, lds);
    if (e != hipSuccess) return e;
    const int row_tiles = (p.M + 15) / 16;
    const int waves = kThreads / kWave;
    int per_slice = device_cu_count() / p.slices;
    const int most = (row_tiles + waves - 1) / waves;
    if (per_slice > most) per_slice = most;
    if (per_slice < 1) per_slice = 1;
    const int64_t grid = (int64_t)per_slice * p.slices;
    e = launch_main(gemm_n_kernel<F, KW>, dim3((unsigned)grid), dim3(kThreads), lds, s, p,
                    per_slice);
    if (e != hipSuccess || p.slices == 1) return e;
    const int64_t nm = (int64_t)p.n * p.M;
    return launch_aux(gemm_n_reduce, dim3((unsigned)((nm + 255) / 256)), dim3(256), 0, s,
                      (const float *)p.partial, p.slices, nm, p.Y);
}

template <class F>
hipError_t launch_typed(const GemmParams &p, hipStream_t s) {
    return windows_per_slice(p.M, p.K) == 2 ? launch_kw<F, 2>(p, s) : launch_kw<F, 1>(p, s);
}

// ---------------------------------------------------------------------------
// Prefill-size product (n up to thousands of tokens; BebeLM page, section
// "性能表现": prompts are processed in batches).  With many tokens there is
// parallelism across token blocks, so K is split only when rows and token
// blocks alone give too few workgroups: a workgroup owns 128 rows, a block
// of 16 * TT tokens and a slice of consecutive 256-weight windows (all of K
// unless split).  Per window it stages X for its tokens (bf16 hi/lo operand
// fragments and per-sub-block sums) in LDS, then multiplies while the next
// window's weights are in flight in a second register set.  Each weight sub-block's codes and scales are formed
// once and used by the TT token tiles.  Two workgroups share a compute unit,
// so one's X staging overlaps the other's multiply.  Every output is one fixed-order sum
// over the windows, or over the slices' partial sums added in slice order by
// a second kernel, so results are deterministic.
// Workgroups are mapped so that those sharing rows run on the same XCD
// (workgroups go to XCDs round-robin): their weights come from that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;

// TT: token tiles of 16 per workgroup (1, 2 or 4, chosen per call so that
// there are enough workgroups)
template <class F, int TT>
struct PfLayout {
    static constexpr int kPfTokens = 16 * TT;
    static constexpr int kVals = F::kNSub * 4 * kPfTokens * F::kKpl;  // = 256 * kPfTokens
    static constexpr int kBytes = kVals * 2 * 2 + F::kNSub * kPfTokens * 4;
};

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
            // lane groups q = 0..3 of (j, t) are lanes tl, tl + 16, tl + 32, tl + 48
            sum += __shfl_xor(sum, 16, kWave);
            sum += __shfl_xor(sum, 32, kWave);
            if (q == 0) reinterpret_cast<float *>(base + 4 * L::kVals)[j * kPfTokens + t] = sum;
        }
    }
};

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
    const BufSrc xview(reinterpret_cast<const uint8_t *>(p.X), (uint64_t)p.n * (uint32_t)p.K * 4u);

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
                const int fo = ((j * 4 + q) * kPfTokens + tt * 16 + r) * F::kKpl;
                const Frag<F> ah = *reinterpret_cast<const Frag<F> *>(xhi + fo);
                const Frag<F> al = *reinterpret_cast<const Frag<F> *>(xlo + fo);
#pragma unroll
                for (int rt = 0; rt < RT; rt++) {
                    f32x4 c = {0.f, 0.f, 0.f, 0.f};
                    c = mfma<F>(ah, bcode[rt], c);
                    c = mfma<F>(al, bcode[rt], c);
                    acc[rt][tt][0] = fmaf(scale[rt], c[0], acc[rt][tt][0]);
                    acc[rt][tt][1] = fmaf(scale[rt], c[1], acc[rt][tt][1]);
                    acc[rt][tt][2] = fmaf(scale[rt], c[2], acc[rt][tt][2]);
                    acc[rt][tt][3] = fmaf(scale[rt], c[3], acc[rt][tt][3]);
                }
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
            XStagePf<F, TT> xs;
            xs.load(xview, p.K, tok0, wi);
            xs.store(smem, wi, p.K);
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
#pragma unroll
    for (int rt = 0; rt < RT; rt++) {
        const int row = row0 + rt * 16 + r;
        if (row < p.M) {
#pragma unroll
            for (int tt = 0; tt < kPfTiles; tt++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int t = tok0 + tt * 16 + 4 * q + i;
                    if (t < p.n) out[(int64_t)t * p.M + row] = acc[rt][tt][i];
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
    if (grid > 0x7FFFFFFFll) return hipErrorInvalidValue;
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

// Prefill launch plan.  The most tokens per workgroup (TT = 4, 2, 1) that
// still gives two workgroups per compute unit of a 256-CU part without a K
// split; failing that, one token tile per workgroup and K split into the
// fewest slices (2 .. 16, at least two windows each) that reach that count.
// The plan depends only on (M, K, n), so the workspace size does too.
PfPlan pf_plan(int64_t M, int64_t K, int64_t n) {
    constexpr int64_t kWant = 512;
    PfPlan pl{};
    const int wtotal = (int)((K + kWin - 1) / kWin);
    auto tblocks = [&](int tt) { return (int)((n + 16 * tt - 1) / (16 * tt)); };
    pl.slices = 1;
    pl.wps = wtotal;
    // two row tiles per wave (256-row workgroups) when that still gives 1.5
    // workgroups per compute unit with 64 tokens each (n = 256 over the 32
    // layers: 17.8 ms with a threshold of 2 per compute unit, 16.8 with 1.5)
    pl.rt = 2;
    pl.tt = 4;
    pl.token_blocks = tblocks(4);
    pl.rg_pad = (int)(((M + 2 * kRowsPerWG - 1) / (2 * kRowsPerWG) + kXcds - 1) / kXcds * kXcds);
    if ((int64_t)pl.rg_pad * pl.token_blocks >= kWant * 3 / 4) return pl;
    pl.rt = 1;
    const int64_t row_groups = (M + kRowsPerWG - 1) / kRowsPerWG;
    pl.rg_pad = (int)((row_groups + kXcds - 1) / kXcds * kXcds);
    for (int tt = 4; tt >= 1; tt >>= 1) {
        pl.tt = tt;
        pl.token_blocks = tblocks(tt);
        if ((int64_t)pl.rg_pad * pl.token_blocks >= kWant) return pl;
    }
    // tt = 1 here
    for (int ks = 2; ks <= 16 && wtotal / ks >= 2; ks *= 2) {
        pl.wps = (wtotal + ks - 1) / ks;
        pl.slices = (wtotal + pl.wps - 1) / pl.wps;  // no empty slice
        if ((int64_t)pl.rg_pad * pl.token_blocks * pl.slices >= kWant) break;
    }
    return pl;
}

size_t gemm_workspace(int64_t M, int64_t K, int64_t n) {
    const PfPlan pl = pf_plan(M, K, n);
    return pl.slices > 1 ? (size_t)pl.slices * (size_t)n * (size_t)M * sizeof(float) : 0;
}

size_t gemm_n_workspace(int64_t M, int64_t K, int32_t n) {
    const int64_t kw = windows_per_slice(M, K);
    const int64_t slices = ((K + kWin - 1) / kWin + kw - 1) / kw;
    return slices > 1 ? (size_t)slices * (size_t)n * (size_t)M * sizeof(float) : 0;
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
    switch (type) {
    case kQ4K: return launch_pf<GQ4K>(p, s);
    case kQ5K: return launch_pf<GQ5K>(p, s);
    case kQ6K: return launch_pf<GQ6K>(p, s);
    case kQ80: return launch_pf<GQ80>(p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_n(int type, const uint8_t *W, int64_t M, int64_t K, int32_t n,
                         const float *X, float *Y, void *ws, hipStream_t s) {
    GemmParams p{};
    p.W = W;
    p.M = (int32_t)M;
    p.K = (int32_t)K;
    p.n = n;
    p.row_bytes = (int32_t)row_bytes_of(type, K);
    p.X = X;
    p.Y = Y;
    p.partial = reinterpret_cast<float *>(ws);
    switch (type) {
    case kQ4K: return launch_typed<GQ4K>(p, s);
    case kQ5K: return launch_typed<GQ5K>(p, s);
    case kQ6K: return launch_typed<GQ6K>(p, s);
    case kQ80: return launch_typed<GQ80>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qmv
