// Shared pieces of the matrix-core products (small-batch verify and
// prefill): bf16 operand types, the per-format weight policies and the MFMA
// helpers.
//
// Exactness plan (the result stays within the f32 matvec's 1e-5 sum|w x|):
//  - the MFMA's weight operand holds the raw integer codes, which bf16
//    represents exactly (written 0x43uu = 128 + u); the f32 scale d*sc is
//    applied to the f32 MFMA result once per sub-block, and the per-sub-block
//    correction (the +128 and the min) times the activation sums is itself a
//    small product, sums[token][j] x corr[j][row], done by one f32 MFMA
//    (16x16x4) per four sub-blocks straight into the accumulator;
//  - X is split into bf16 hi + lo, so the only representation error is
//    |x - hi - lo| <= 2^-18 |x|.
// Operand roles: tokens (or token halves) are the MFMA M side (A = X
// fragment), weight rows the N side (B = codes), so a lane's accumulators all
// belong to the row whose block header that lane loaded and the scales apply
// lane-locally.
//   v_mfma_f32_16x16x32_bf16 (Q4_K, Q5_K, Q8_0: one 32-weight sub-block /
//   block) and v_mfma_f32_16x16x16_bf16 (Q6_K: one 16-weight sub-block);
//   lane l of a wave supplies A[l%16][kpl*(l/16) + t], B[kpl*(l/16) + t][l%16]
//   and holds C[4*(l/16) + i][l%16].
#pragma once

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
    uint8_t *xprep;    // activations in the staged operand layout (prefill)
    int32_t row_groups;
    int32_t slices;
    int32_t windows;   // 256-weight windows of K
};

constexpr int kThreads = 512;  // 8 waves
constexpr int kRowsPerWG = 128;

// ---------------------------------------------------------------------------
// Cross-row moves.  In the operand layout the four lanes that share a weight
// row (r, r + 16, r + 32, r + 48) sit in the wave's four 16-lane rows, and
// neighbouring lanes belong to different weight rows, so a load that gives
// each lane only the bytes of its own k-slots costs the L1 one request per
// lane.  The fetches below instead give each lane whole 16-byte pieces of its
// row and exchange dwords between the four rows with gfx950's row swaps
// (v_permlane32_swap: upper 32 lanes of one register <-> lower 32 lanes of
// another; v_permlane16_swap: odd 16-lane rows of one <-> even rows of
// another).  Every lane of the wave must be active.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void as_words(uint32_t (&w)[4], const uint4 &v) {
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
}
// 4 x 4 transpose over the rows: afterwards v[c] in row q is what v[q] held
// in row c (each lane keeps its position within the row).
__device__ __forceinline__ void xpose_rows(uint32_t (&v)[4]) {
    const auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    v[0] = c[0];
    v[1] = c[1];
    v[2] = d[0];
    v[3] = d[1];
}
// Sum of v over the four rows, the same bits in every row ((r0 + r1) + (r2 + r3)).
// (The swap results are copied out element by element: a bit cast applied
// straight to an element of the returned vector reads element 0.)
__device__ __forceinline__ float rows_sum(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // (0,0,2,2) | (1,1,3,3)
    const uint32_t a0 = a[0], a1 = a[1];
    const float t = __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1);
    const uint32_t tu = __builtin_bit_cast(uint32_t, t);
    const auto b = __builtin_amdgcn_permlane32_swap(tu, tu, false, false);  // (01 x4) | (23 x4)
    const uint32_t b0 = b[0], b1 = b[1];
    return __builtin_bit_cast(float, b0) + __builtin_bit_cast(float, b1);
}
// What row 0 (ROW = 0) or row 1 (ROW = 1) of v holds, in every row.
template <int ROW>
__device__ __forceinline__ uint32_t row_bcast(uint32_t v) {
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // (0,0,2,2) | (1,1,3,3)
    const uint32_t e = a[ROW];
    return __builtin_amdgcn_permlane32_swap(e, e, false, false)[0];      // rows 0,1 copied up
}

// ---------------------------------------------------------------------------
// Format policies.  kSub: weights per MFMA sub-block (= MFMA K); kNSub:
// sub-blocks per 256-weight window; kKpl: operand values per lane.
// slot(i): where weight i (0..255) of a window sits in the operand layout, as
// (sub-block j, lane group q, slot t).  load(src, off, q, nvalid): the bytes
// lane group q needs from the window starting `off` bytes into the view;
// fetch(...) issues wider loads of the same bytes into a Wide set, and
// regs(wide) rearranges it into the Regs that load returns.
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
    // The same bytes from wide loads (fetch, at issue time) and a transpose
    // (regs, at use time): lane group q reads nibble chunk q whole, two
    // 16-byte loads, and the 8-byte pieces move across the groups, low and
    // high dwords separately.
    struct Wide {
        uint4 hdr, a, b;
    };
    __device__ static Wide fetch(const BufSrc &src, uint32_t off, int q, int) {
        Wide w;
        w.hdr = src.ld16(off);
        w.a = src.ld16(off + 16 + 32 * q);
        w.b = src.ld16(off + 32 + 32 * q);
        return w;
    }
    __device__ static void pieces_of(uint2 (&piece)[4], const uint4 &a, const uint4 &b) {
        uint32_t lo[4] = {a.x, a.z, b.x, b.z}, hi[4] = {a.y, a.w, b.y, b.w};
        xpose_rows(lo);
        xpose_rows(hi);
#pragma unroll
        for (int c = 0; c < 4; c++) piece[c] = make_uint2(lo[c], hi[c]);
    }
    __device__ static Regs regs(const Wide &w) {
        Regs r;
        r.hdr = w.hdr;
        pieces_of(r.piece, w.a, w.b);
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
    // The correction of sub-block j0 + q (j0 = 0 or 4, fixed where the
    // caller's loop unrolls; q the lane group, 0..3), without the selects
    // that a lane-dependent sub-block index costs: the same value as
    // corr_of(r, j0 + q).
    __device__ static float corr_q(const Regs &r, int j0, int q) { return hdr_corr_q(r.hdr, j0, q); }
    __device__ static float hdr_corr_q(const uint4 &hdr, int j0, int q) {
        const uint32_t sh = 8u * (uint32_t)q;
        const uint32_t y = hdr.y >> sh, z = hdr.z >> sh, w = hdr.w >> sh;
        int sc, m;
        if (j0 == 0) {
            sc = (int)(y & 63u);
            m = (int)(z & 63u);
        } else {
            sc = (int)((w & 15u) | (((y >> 6) & 3u) << 4));
            m = (int)(((w >> 4) & 15u) | (((z >> 6) & 3u) << 4));
        }
        const float dmin = half_bits_to_float(hdr.x >> 16);
        return fmaf(128.0f, half_bits_to_float(hdr.x) * (float)sc, dmin * (float)m);
    }
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
    struct Wide {
        uint4 hdr;
        uint2 qh;
        uint4 a, b;
    };
    __device__ static Wide fetch(const BufSrc &src, uint32_t off, int q, int) {
        Wide w;
        w.hdr = src.ld16(off);
        w.qh = src.ld8(off + 16 + 8 * q);
        w.a = src.ld16(off + 48 + 32 * q);
        w.b = src.ld16(off + 64 + 32 * q);
        return w;
    }
    __device__ static Regs regs(const Wide &w) {
        Regs r;
        r.hdr = w.hdr;
        r.qh = w.qh;
        GQ4K::pieces_of(r.piece, w.a, w.b);
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
    __device__ static float corr_q(const Regs &r, int j0, int q) { return GQ4K::hdr_corr_q(r.hdr, j0, q); }
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
    // The same registers from four 16-byte loads per lane: group q reads QL
    // chunks q and 4 + q and QH chunk q, transposed across the groups; group
    // 0 reads the scales, group 1 the 16 bytes ending with d, and both are
    // copied to every group.
    struct Wide {
        uint4 a, b, c, e;
    };
    __device__ static Wide fetch(const BufSrc &src, uint32_t off, int q, int) {
        Wide w;
        w.a = src.ld16(off + 16 * q);
        w.b = src.ld16(off + 64 + 16 * q);
        w.c = src.ld16(off + 128 + 16 * q);
        w.e = src.ld16(off + 192 + 2 * (q & 1));
        return w;
    }
    __device__ static Regs regs(const Wide &w) {
        uint32_t a[4], b[4], c[4], e[4];
        as_words(a, w.a);
        as_words(b, w.b);
        as_words(c, w.c);
        as_words(e, w.e);
        xpose_rows(a);
        xpose_rows(b);
        xpose_rows(c);
        Regs r;
#pragma unroll
        for (int g = 0; g < 2; g++)
#pragma unroll
            for (int hh = 0; hh < 2; hh++) {
                r.ql[0][g][hh] = a[2 * g + hh];
                r.ql[1][g][hh] = b[2 * g + hh];
                r.qh[g][hh] = c[2 * g + hh];
            }
        r.sc = make_uint4(row_bcast<0>(e[0]), row_bcast<0>(e[1]), row_bcast<0>(e[2]),
                          row_bcast<0>(e[3]));
        r.d = row_bcast<1>(e[3]) >> 16;
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
    // corr_of(r, j0 + q) for j0 a multiple of 4 and q < 4
    __device__ static float corr_q(const Regs &r, int j0, int q) {
        const uint32_t w = j0 < 4 ? r.sc.x : j0 < 8 ? r.sc.y : j0 < 12 ? r.sc.z : r.sc.w;
        const float s = half_bits_to_float(r.d) * (float)(int32_t)(int8_t)((w >> (8 * q)) & 0xFFu);
        return 160.0f * s;
    }
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
    // (no wide form: the blocks' 34-byte stride does not split into
    // 16-byte pieces)
    using Wide = Regs;
    __device__ static Wide fetch(const BufSrc &src, uint32_t off, int q, int nvalid) {
        return load(src, off, q, nvalid);
    }
    __device__ static Regs regs(const Wide &w) { return w; }
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
    __device__ static float corr_q(const Regs &, int, int) { return 0.f; }
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
    const float b = F::corr_q(w, j0, q);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

template <class F>
__device__ __forceinline__ f32x4 mfma(const Frag<F> &a, const Frag<F> &b, f32x4 c) {
    if constexpr (F::kKpl == 8)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

}  // namespace

}  // namespace qmv
