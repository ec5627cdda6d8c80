// Per-format "unit" decoders for the gfx950 matvec kernels.
//
// A unit is the slice of one row that one lane handles per step: 64 weights
// (32 for Q8_0 rows with an odd number of blocks).  Lanes keep the same unit
// position modulo 4 for a whole launch, so the sub-block they touch inside a
// 256-weight super-block is lane-constant.  Each decoder
//   - loads its unit's bytes straight from HBM with 128-bit buffer loads
//     (load; `off` is the byte offset of the unit's region, unit_offset),
//   - reads the unit's 64 activations from LDS (load_x),
//   - multiplies and adds into a per-lane f32 accumulator (dot), using the
//     factored form  d*sc_j*sum(q*x) - dmin*m_j*sum(x)  so that the scales are
//     applied once per 16 or 32 weights, never per weight.
//
// Block layouts (bytes, little-endian), standard GGUF bit order:
//   Q8_0 34 B / 32 w:  fp16 d | int8 q[32]
//   Q4_K 144 B / 256 w: fp16 d | fp16 dmin | S[12] (6-bit sc/m of 8 sub-blocks)
//                      | Q[128]: byte 32c+l holds weight 64c+l (low nibble)
//                        and weight 64c+32+l (high nibble)
//   Q6_K 210 B / 256 w: QL[128] | QH[64] | int8 sc[16] | fp16 d; weight
//                      128n+32g+l takes its low 4 bits from QL[64n+l+32(g&1)]
//                      (nibble g>>1) and its high 2 bits from bits 2g..2g+1 of
//                      QH[32n+l]; q - 32 is the signed code, sub-block = i/16.
// BebeLM page ("BebeLM：纯Rust实现的端侧大模型推理引擎"), section "量化格式支持"
// (Q4_K: 256 weights in 144 bytes; Q6_K for sensitive tensors; f32
// activations); Wick page, section "量化支持" (Q8_0).
#pragma once

#include "qmv_device.h"

namespace qmv {

// ---------------------------------------------------------------------------
// Q4_K: unit u of a row = block u/4, 64-weight chunk c = u%4, i.e. nibble
// bytes Q[32c .. 32c+32): low nibbles are sub-block 2c, high nibbles 2c+1.
// Activation sums per 32-weight sub-block come from LDS (`sums`).
// ---------------------------------------------------------------------------
struct Q4K {
    static constexpr int kBlockWeights = 256;
    static constexpr int kBlockBytes = 144;
    static constexpr int kUnitWeights = 64;
    static constexpr int kSumGroup = 32;  // activation sums per sub-block of 32
    static constexpr int kPadEvery = 64;  // LDS copy of x: 4 pad floats per 64
    struct Regs {
        uint4 hdr, q0, q1;
    };
    __device__ static __forceinline__ uint32_t unit_offset(int u) {
        return (uint32_t)(u >> 2) * kBlockBytes;
    }
    __device__ static __forceinline__ Regs load(const BufSrc &src, uint32_t off, int u) {
        const uint32_t c = u & 3;
        Regs r;
        r.hdr = src.ld16(off);
        r.q0 = src.ld16(off + 16 + 32 * c);
        r.q1 = src.ld16(off + 32 + 32 * c);
        return r;
    }
    // The unit's 64 activations: x[64u .. 64u+64), stored at 68u in the padded
    // LDS copy, so lane u's i-th 16-byte read falls in bank group (u + i) mod 16
    // and consecutive lanes never collide.
    __device__ static __forceinline__ void load_x(const float *xs, int u, float *xv) {
        const float4 *p = reinterpret_cast<const float4 *>(xs + 68 * u);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            float4 v = p[i];
            xv[4 * i] = v.x;
            xv[4 * i + 1] = v.y;
            xv[4 * i + 2] = v.z;
            xv[4 * i + 3] = v.w;
        }
    }
    // acc += sum over the unit's 64 weights of w * x.  Byte 32c + l of the
    // unit's nibbles holds weight l (low nibble) and weight 32 + l (high
    // nibble) of sub-blocks 2c and 2c + 1.  A dword of four such bytes,
    // masked in place, holds the low nibbles of bytes 0 and 2 as two f16
    // subnormals q * 2^-24 (and their high nibbles as 16 q * 2^-24); the
    // dword shifted right by 8 gives bytes 1 and 3 the same way.  That is
    // one shift and four masks per eight weights.
    __device__ static __forceinline__ void dot(const Regs &r, const float *xv, const float *sums,
                                               int u, float &acc) {
        const uint32_t qw[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
        float lo0 = 0.f, lo1 = 0.f, hi0 = 0.f, hi1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t w = qw[i], w8 = qw[i] >> 8;
            const f16x2_t a02 = as_f16x2(w & 0x000F000Fu), a13 = as_f16x2(w8 & 0x000F000Fu);
            const f16x2_t b02 = as_f16x2(w & 0x00F000F0u), b13 = as_f16x2(w8 & 0x00F000F0u);
            lo0 = fmaf((float)a02.x, xv[4 * i + 0], lo0);
            lo1 = fmaf((float)a02.y, xv[4 * i + 2], lo1);
            lo0 = fmaf((float)a13.x, xv[4 * i + 1], lo0);
            lo1 = fmaf((float)a13.y, xv[4 * i + 3], lo1);
            hi0 = fmaf((float)b02.x, xv[32 + 4 * i + 0], hi0);
            hi1 = fmaf((float)b02.y, xv[32 + 4 * i + 2], hi1);
            hi0 = fmaf((float)b13.x, xv[32 + 4 * i + 1], hi0);
            hi1 = fmaf((float)b13.y, xv[32 + 4 * i + 3], hi1);
        }
        // both sums at the scale 2^-24 (the high nibbles carried 16 q)
        const float alo = lo0 + lo1, ahi = (hi0 + hi1) * 0.0625f;
        // 6-bit scale and min of sub-blocks 2c and 2c+1, as two bytes each
        // (both decodings are formed and one is selected: no branch).
        const int c = u & 3;
        const int sh = (c & 1) * 16;
        const uint32_t s0 = r.hdr.y >> sh, s1 = r.hdr.z >> sh, s2 = r.hdr.w >> sh;
        const uint32_t sc_lo = s0 & 0x3F3Fu, m_lo = s1 & 0x3F3Fu;
        const uint32_t sc_hi = (s2 & 0x0F0Fu) | ((s0 >> 2) & 0x3030u);
        const uint32_t m_hi = ((s2 >> 4) & 0x0F0Fu) | ((s1 >> 2) & 0x3030u);
        const uint32_t sc = c < 2 ? sc_lo : sc_hi;
        const uint32_t m = c < 2 ? m_lo : m_hi;
        const float d = half_bits_to_float(r.hdr.x) * kTwo24;
        const float dmin = half_bits_to_float(r.hdr.x >> 16);
        const float t = fmaf(ubyte<1>(sc), ahi, ubyte<0>(sc) * alo);
        const float mm = fmaf(ubyte<1>(m), sums[2 * u + 1], ubyte<0>(m) * sums[2 * u]);
        acc = fmaf(d, t, acc);
        acc = fmaf(-dmin, mm, acc);
    }
};

// ---------------------------------------------------------------------------
// Q6_K: unit u of a row = block u/4, half n = (u>>1)&1, h = u&1: weights
// 128n + 32g + 16h + t for g, t in 0..3 x 0..15 (sub-blocks 8n+2g+h).
// Activation sums per 16-weight sub-block come from LDS; the -32 offset of
// the codes is applied through them.
// ---------------------------------------------------------------------------
struct Q6K {
    static constexpr int kBlockWeights = 256;
    static constexpr int kBlockBytes = 210;
    static constexpr int kUnitWeights = 64;
    static constexpr int kSumGroup = 16;
    static constexpr int kPadEvery = 128;  // LDS copy of x: 4 pad floats per 128
    struct Regs {
        uint4 qa, qb, qh;
        uint2 sc;
        uint32_t d;
    };
    __device__ static __forceinline__ uint32_t unit_offset(int u) {
        return (uint32_t)(u >> 2) * kBlockBytes;
    }
    __device__ static __forceinline__ Regs load(const BufSrc &src, uint32_t off, int u) {
        const uint32_t n = (u >> 1) & 1, h = u & 1;
        Regs r;
        r.qa = src.ld16(off + 64 * n + 16 * h);
        r.qb = src.ld16(off + 64 * n + 32 + 16 * h);
        r.qh = src.ld16(off + 128 + 32 * n + 16 * h);
        r.sc = src.ld8(off + 192 + 8 * n);
        r.d = src.ld2(off + 208);
        return r;
    }
    // Runs x[256b + 128n + 32g + 16h .. +16) for g = 0..3; in the padded LDS
    // copy (4 pad floats per 128) the 8 units of two blocks start in 8
    // distinct bank groups.
    __device__ static __forceinline__ void load_x(const float *xs, int u, float *xv) {
        const int b = u >> 2, n = (u >> 1) & 1, h = u & 1;
        const float *base = xs + 264 * b + 132 * n + 16 * h;
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const float4 *p = reinterpret_cast<const float4 *>(base + 32 * g);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float4 v = p[i];
                xv[16 * g + 4 * i] = v.x;
                xv[16 * g + 4 * i + 1] = v.y;
                xv[16 * g + 4 * i + 2] = v.z;
                xv[16 * g + 4 * i + 3] = v.w;
            }
        }
    }
    // The 6-bit codes of four sub-blocks are assembled bytewise, then spread
    // two per dword into f16 subnormals (q * 2^-24) for the multiply-adds.
    __device__ static __forceinline__ void dot(const Regs &r, const float *xv, const float *sums,
                                               int u, float &acc) {
        const uint32_t qa[4] = {r.qa.x, r.qa.y, r.qa.z, r.qa.w};
        const uint32_t qb[4] = {r.qb.x, r.qb.y, r.qb.z, r.qb.w};
        const uint32_t qh[4] = {r.qh.x, r.qh.y, r.qh.z, r.qh.w};
        float A[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t a = qa[i], b = qb[i], hh = qh[i];
            const uint32_t q[4] = {
                (a & 0x0F0F0F0Fu) | ((hh & 0x03030303u) << 4),
                (b & 0x0F0F0F0Fu) | ((hh & 0x0C0C0C0Cu) << 2),
                ((a >> 4) & 0x0F0F0F0Fu) | (hh & 0x30303030u),
                ((b >> 4) & 0x0F0F0F0Fu) | ((hh >> 2) & 0x30303030u),
            };
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const f16x2_t c01 = as_f16x2(bytes01_to_halves(q[g]));
                const f16x2_t c23 = as_f16x2(bytes23_to_halves(q[g]));
                A[g] = fmaf((float)c01.x, xv[16 * g + 4 * i + 0], A[g]);
                A[g] = fmaf((float)c01.y, xv[16 * g + 4 * i + 1], A[g]);
                A[g] = fmaf((float)c23.x, xv[16 * g + 4 * i + 2], A[g]);
                A[g] = fmaf((float)c23.y, xv[16 * g + 4 * i + 3], A[g]);
            }
        }
        // sub-block of group g is 8n + 2g + h: its scale is byte 2g + h of the
        // 8 scale bytes loaded from 192 + 8n; its activation sum is entry
        // 16*b + 8n + 2g + h of `sums`.
        const int h = u & 1;
        const int sbase = 16 * (u >> 2) + 8 * ((u >> 1) & 1) + h;
        const uint32_t w0 = r.sc.x >> (8 * h), w1 = r.sc.y >> (8 * h);
        float t = 0.f;
        // A[g] * 2^24 is the code sum exactly (power-of-two scaling)
        t = fmaf(sbyte<0>(w0), fmaf(A[0], kTwo24, -32.f * sums[sbase + 0]), t);
        t = fmaf(sbyte<2>(w0), fmaf(A[1], kTwo24, -32.f * sums[sbase + 2]), t);
        t = fmaf(sbyte<0>(w1), fmaf(A[2], kTwo24, -32.f * sums[sbase + 4]), t);
        t = fmaf(sbyte<2>(w1), fmaf(A[3], kTwo24, -32.f * sums[sbase + 6]), t);
        acc = fmaf(half_bits_to_float(r.d), t, acc);
    }
};

// ---------------------------------------------------------------------------
// Q8_0, two blocks per unit (rows with an even number of blocks): unit u =
// blocks 2u and 2u+1 = 68 bytes starting 68u into the row (4-byte aligned).
// ---------------------------------------------------------------------------
struct Q80x2 {
    static constexpr int kBlockWeights = 32;
    static constexpr int kBlockBytes = 34;
    static constexpr int kUnitWeights = 64;
    static constexpr int kSumGroup = 0;
    static constexpr int kPadEvery = 64;
    struct Regs {
        uint4 a, b, c, d;
        uint32_t e;
    };
    __device__ static __forceinline__ uint32_t unit_offset(int u) { return (uint32_t)u * 68; }
    __device__ static __forceinline__ Regs load(const BufSrc &src, uint32_t off, int) {
        Regs r;
        r.a = src.ld16(off);
        r.b = src.ld16(off + 16);
        r.c = src.ld16(off + 32);
        r.d = src.ld16(off + 48);
        r.e = src.ld4(off + 64);
        return r;
    }
    __device__ static __forceinline__ void load_x(const float *xs, int u, float *xv) {
        Q4K::load_x(xs, u, xv);
    }
    __device__ static __forceinline__ void dot(const Regs &r, const float *xv, const float *,
                                               int, float &acc) {
        const uint32_t D[17] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w,
                                r.c.x, r.c.y, r.c.z, r.c.w, r.d.x, r.d.y, r.d.z, r.d.w, r.e};
        // block 0: d in D0 bytes 0-1, q[0..1] in D0 bytes 2-3, q[2..29] in
        // D1..D7, q[30..31] in D8 bytes 0-1.  Block 1: d in D8 bytes 2-3,
        // q[0..31] in D9..D16.
        float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
        a0 = fmaf(sbyte<2>(D[0]), xv[0], a0);
        a1 = fmaf(sbyte<3>(D[0]), xv[1], a1);
#pragma unroll
        for (int i = 1; i < 8; i++) {
            a0 = fmaf(sbyte<0>(D[i]), xv[4 * i - 2], a0);
            a1 = fmaf(sbyte<1>(D[i]), xv[4 * i - 1], a1);
            a0 = fmaf(sbyte<2>(D[i]), xv[4 * i + 0], a0);
            a1 = fmaf(sbyte<3>(D[i]), xv[4 * i + 1], a1);
        }
        a0 = fmaf(sbyte<0>(D[8]), xv[30], a0);
        a1 = fmaf(sbyte<1>(D[8]), xv[31], a1);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            b0 = fmaf(sbyte<0>(D[9 + i]), xv[32 + 4 * i + 0], b0);
            b1 = fmaf(sbyte<1>(D[9 + i]), xv[32 + 4 * i + 1], b1);
            b0 = fmaf(sbyte<2>(D[9 + i]), xv[32 + 4 * i + 2], b0);
            b1 = fmaf(sbyte<3>(D[9 + i]), xv[32 + 4 * i + 3], b1);
        }
        acc = fmaf(half_bits_to_float(D[0]), a0 + a1, acc);
        acc = fmaf(half_bits_to_float(D[8] >> 16), b0 + b1, acc);
    }
};

// ---------------------------------------------------------------------------
// Q8_0, one block per unit (any row length): 34 bytes at 34u, 2-byte aligned.
// ---------------------------------------------------------------------------
struct Q80x1 {
    static constexpr int kBlockWeights = 32;
    static constexpr int kBlockBytes = 34;
    static constexpr int kUnitWeights = 32;
    static constexpr int kSumGroup = 0;
    static constexpr int kPadEvery = 32;
    struct Regs {
        uint4 a, b;
        uint32_t c;
    };
    __device__ static __forceinline__ uint32_t unit_offset(int u) { return (uint32_t)u * 34; }
    __device__ static __forceinline__ Regs load(const BufSrc &src, uint32_t off, int) {
        Regs r;
        r.c = src.ld2(off);
        r.a = src.ld16(off + 2);
        r.b = src.ld16(off + 18);
        return r;
    }
    __device__ static __forceinline__ void load_x(const float *xs, int u, float *xv) {
        const float4 *p = reinterpret_cast<const float4 *>(xs + 36 * u);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float4 v = p[i];
            xv[4 * i] = v.x;
            xv[4 * i + 1] = v.y;
            xv[4 * i + 2] = v.z;
            xv[4 * i + 3] = v.w;
        }
    }
    __device__ static __forceinline__ void dot(const Regs &r, const float *xv, const float *,
                                               int, float &acc) {
        const uint32_t D[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            a0 = fmaf(sbyte<0>(D[i]), xv[4 * i + 0], a0);
            a1 = fmaf(sbyte<1>(D[i]), xv[4 * i + 1], a1);
            a0 = fmaf(sbyte<2>(D[i]), xv[4 * i + 2], a0);
            a1 = fmaf(sbyte<3>(D[i]), xv[4 * i + 3], a1);
        }
        acc = fmaf(half_bits_to_float(r.c), a0 + a1, acc);
    }
};

// ---------------------------------------------------------------------------
// Q5_K (BebeLM page, section "局限与未来": Q5_K_M): the Q4_K super-block plus
// 32 bytes of fifth bits.  Unit u = chunk c = u & 3 of block u / 4, as in
// Q4_K: weights 64c + l (low nibble of byte 32c + l, fifth bit 2c of high
// byte l) and 64c + 32 + l (high nibble, fifth bit 2c + 1).  The 5-bit codes
// are assembled bytewise, then spread two per dword into f16 subnormals.
// ---------------------------------------------------------------------------
struct Q5K {
    static constexpr int kBlockWeights = 256;
    static constexpr int kBlockBytes = 176;
    static constexpr int kUnitWeights = 64;
    static constexpr int kSumGroup = 32;
    static constexpr int kPadEvery = 64;
    struct Regs {
        uint4 hdr, q0, q1, h0, h1;
    };
    __device__ static __forceinline__ uint32_t unit_offset(int u) {
        return (uint32_t)(u >> 2) * kBlockBytes;
    }
    __device__ static __forceinline__ Regs load(const BufSrc &src, uint32_t off, int u) {
        const uint32_t c = u & 3;
        Regs r;
        r.hdr = src.ld16(off);
        r.h0 = src.ld16(off + 16);
        r.h1 = src.ld16(off + 32);
        r.q0 = src.ld16(off + 48 + 32 * c);
        r.q1 = src.ld16(off + 64 + 32 * c);
        return r;
    }
    __device__ static __forceinline__ void load_x(const float *xs, int u, float *xv) {
        Q4K::load_x(xs, u, xv);
    }
    __device__ static __forceinline__ void dot(const Regs &r, const float *xv, const float *sums,
                                               int u, float &acc) {
        const uint32_t qw[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
        const uint32_t hw[8] = {r.h0.x, r.h0.y, r.h0.z, r.h0.w, r.h1.x, r.h1.y, r.h1.z, r.h1.w};
        const int c = u & 3;
        float lo0 = 0.f, lo1 = 0.f, hi0 = 0.f, hi1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t t = hw[i] >> (2 * c);
            const uint32_t a = (qw[i] & 0x0F0F0F0Fu) | ((t & 0x01010101u) << 4);
            const uint32_t b = ((qw[i] >> 4) & 0x0F0F0F0Fu) | ((t & 0x02020202u) << 3);
            const f16x2_t a01 = as_f16x2(bytes01_to_halves(a)), a23 = as_f16x2(bytes23_to_halves(a));
            const f16x2_t b01 = as_f16x2(bytes01_to_halves(b)), b23 = as_f16x2(bytes23_to_halves(b));
            lo0 = fmaf((float)a01.x, xv[4 * i + 0], lo0);
            lo1 = fmaf((float)a01.y, xv[4 * i + 1], lo1);
            lo0 = fmaf((float)a23.x, xv[4 * i + 2], lo0);
            lo1 = fmaf((float)a23.y, xv[4 * i + 3], lo1);
            hi0 = fmaf((float)b01.x, xv[32 + 4 * i + 0], hi0);
            hi1 = fmaf((float)b01.y, xv[32 + 4 * i + 1], hi1);
            hi0 = fmaf((float)b23.x, xv[32 + 4 * i + 2], hi0);
            hi1 = fmaf((float)b23.y, xv[32 + 4 * i + 3], hi1);
        }
        const float alo = lo0 + lo1, ahi = hi0 + hi1;  // at the scale 2^-24
        // 6-bit scales and mins of sub-blocks 2c and 2c + 1 (the Q4_K packing)
        const int sh = (c & 1) * 16;
        const uint32_t s0 = r.hdr.y >> sh, s1 = r.hdr.z >> sh, s2 = r.hdr.w >> sh;
        const uint32_t sc_lo = s0 & 0x3F3Fu, m_lo = s1 & 0x3F3Fu;
        const uint32_t sc_hi = (s2 & 0x0F0Fu) | ((s0 >> 2) & 0x3030u);
        const uint32_t m_hi = ((s2 >> 4) & 0x0F0Fu) | ((s1 >> 2) & 0x3030u);
        const uint32_t sc = c < 2 ? sc_lo : sc_hi;
        const uint32_t m = c < 2 ? m_lo : m_hi;
        const float d = half_bits_to_float(r.hdr.x) * kTwo24;
        const float dmin = half_bits_to_float(r.hdr.x >> 16);
        const float t = fmaf(ubyte<1>(sc), ahi, ubyte<0>(sc) * alo);
        const float mm = fmaf(ubyte<1>(m), sums[2 * u + 1], ubyte<0>(m) * sums[2 * u]);
        acc = fmaf(d, t, acc);
        acc = fmaf(-dmin, mm, acc);
    }
};

// ---------------------------------------------------------------------------
// Q2_K and Q3_K (FlareLLM page, section "量化技术的全面支持": K-quants from
// Q2K up).  Both store 256 weights as 2-bit codes Q[64], byte 32n + l
// holding weight 128n + 32p + l in bits 2p..2p+1, with 16-weight sub-blocks
// j = i / 16.  The unit is the Q6_K one: half n = (u >> 1) & 1, h = u & 1,
// weights 128n + 32p + 16h + t for p, t in 0..3 x 0..15, i.e. the 16 code
// bytes Q[32n + 16h ..) and sub-blocks 8n + 2p + h.  Plane p of a code dword
// is masked in place, so its bytes are a power-of-two multiple of the code;
// that power is undone with the sub-block scale.
// ---------------------------------------------------------------------------
struct LowBitK {
    static constexpr int kBlockWeights = 256;
    static constexpr int kUnitWeights = 64;
    static constexpr int kSumGroup = 16;
    static constexpr int kPadEvery = 128;
    __device__ static __forceinline__ uint32_t half_of(int u) { return (u >> 1) & 1; }
    __device__ static __forceinline__ void load_x(const float *xs, int u, float *xv) {
        Q6K::load_x(xs, u, xv);
    }
    // A[p] += sum over the 16 weights of plane p of (2^e c) 2^-24 x, where
    // code bytes c come from `plane(i, p)` (dword i = weights t = 4i..4i+3).
    template <class Plane>
    __device__ static __forceinline__ void planes(const float *xv, Plane plane, float *A) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
#pragma unroll
            for (int p = 0; p < 4; p++) {
                const uint32_t c = plane(i, p);
                const f16x2_t c01 = as_f16x2(bytes01_to_halves(c));
                const f16x2_t c23 = as_f16x2(bytes23_to_halves(c));
                A[p] = fmaf((float)c01.x, xv[16 * p + 4 * i + 0], A[p]);
                A[p] = fmaf((float)c01.y, xv[16 * p + 4 * i + 1], A[p]);
                A[p] = fmaf((float)c23.x, xv[16 * p + 4 * i + 2], A[p]);
                A[p] = fmaf((float)c23.y, xv[16 * p + 4 * i + 3], A[p]);
            }
        }
    }
};

// Q2_K, 84 B: S[16] (scale in the low, min in the high nibble of sub-block
// j's byte) | Q[64] | fp16 d | fp16 dmin.  w = d*sc_j*q - dmin*m_j.
struct Q2K : LowBitK {
    static constexpr int kBlockBytes = 84;
    struct Regs {
        uint4 q;
        uint2 sm;     // S[8n .. 8n + 8)
        uint32_t dd;  // d | dmin << 16
    };
    __device__ static __forceinline__ uint32_t unit_offset(int u) {
        return (uint32_t)(u >> 2) * kBlockBytes;
    }
    __device__ static __forceinline__ Regs load(const BufSrc &src, uint32_t off, int u) {
        const uint32_t n = half_of(u), h = u & 1;
        Regs r;
        r.q = src.ld16(off + 16 + 32 * n + 16 * h);
        r.sm = src.ld8(off + 8 * n);
        r.dd = src.ld4(off + 80);
        return r;
    }
    __device__ static __forceinline__ void dot(const Regs &r, const float *xv, const float *sums,
                                               int u, float &acc) {
        const uint32_t qw[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
        float A[4] = {0.f, 0.f, 0.f, 0.f};
        planes(xv, [&](int i, int p) { return qw[i] & (0x03030303u << (2 * p)); }, A);
        // sub-block of plane p is 8n + 2p + h: byte 2p + h of S[8n ..)
        const int h = u & 1;
        const int sbase = 16 * (u >> 2) + 8 * (int)half_of(u) + h;
        const uint32_t w0 = r.sm.x >> (8 * h), w1 = r.sm.y >> (8 * h);
        const uint32_t b[4] = {w0, w0 >> 16, w1, w1 >> 16};
        float t = 0.f, mm = 0.f;
#pragma unroll
        for (int p = 0; p < 4; p++) {
            // A[p] 2^24 / 4^p is the code sum exactly (power-of-two scaling)
            const float sc = (float)(b[p] & 15u) * (kTwo24 / (float)(1 << (2 * p)));
            t = fmaf(sc, A[p], t);
            mm = fmaf((float)((b[p] >> 4) & 15u), sums[sbase + 2 * p], mm);
        }
        acc = fmaf(half_bits_to_float(r.dd), t, acc);
        acc = fmaf(-half_bits_to_float(r.dd >> 16), mm, acc);
    }
};

// Q3_K, 110 B: H[32] | Q[64] | S[12] (6-bit scales, stored + 32) | fp16 d.
// Weight 128n + 32p + l: low bits from Q, bit 4n + p of H[l] set keeps the
// code, clear lowers it by 4.  With c = low | hbit << 2 (0..7) the code is
// c - 4; the -4 is applied through the sub-block activation sums.
// Scale of sub-block j: low four bits from nibble j / 8 of S[j % 8], top two
// from bits 2(j / 4).. of S[8 + j % 4]; for this unit's j = 8n + 2p + h that
// is nibble n of S[2p + h] and bits 2(2n + p / 2) of S[8 + 2(p & 1) + h].
struct Q3K : LowBitK {
    static constexpr int kBlockBytes = 110;
    struct Regs {
        uint4 q, hb;
        uint2 slo;     // S[0 .. 8)
        uint32_t shi;  // S[8 .. 12)
        uint32_t d;
    };
    __device__ static __forceinline__ uint32_t unit_offset(int u) {
        return (uint32_t)(u >> 2) * kBlockBytes;
    }
    __device__ static __forceinline__ Regs load(const BufSrc &src, uint32_t off, int u) {
        const uint32_t n = half_of(u), h = u & 1;
        Regs r;
        r.q = src.ld16(off + 32 + 32 * n + 16 * h);
        r.hb = src.ld16(off + 16 * h);
        r.slo = src.ld8(off + 96);
        r.shi = src.ld4(off + 104);
        r.d = src.ld2(off + 108);
        return r;
    }
    __device__ static __forceinline__ void dot(const Regs &r, const float *xv, const float *sums,
                                               int u, float &acc) {
        const int n = (int)half_of(u), h = u & 1;
        const uint32_t qw[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
        // high bits of this half moved to bits 0..3 of each byte
        const uint32_t hw[4] = {r.hb.x >> (4 * n), r.hb.y >> (4 * n), r.hb.z >> (4 * n),
                                r.hb.w >> (4 * n)};
        // Plane p's 3-bit code is kept at bits e..e+2 of its byte, e = 2p for
        // p < 3; plane 3 would reach bit 8, so its low bits are shifted down
        // to bits 4..5 (e = 4).
        float A[4] = {0.f, 0.f, 0.f, 0.f};
        planes(xv, [&](int i, int p) {
            if (p < 3)
                return (qw[i] & (0x03030303u << (2 * p))) |
                       ((hw[i] & (0x01010101u << p)) << (p + 2));
            return ((qw[i] >> 2) & 0x30303030u) | ((hw[i] & 0x08080808u) << 3);
        }, A);
        const int sbase = 16 * (u >> 2) + 8 * n + h;
        const uint32_t lo0 = r.slo.x >> (8 * h + 4 * n), lo1 = r.slo.y >> (8 * h + 4 * n);
        const uint32_t lo[4] = {lo0, lo0 >> 16, lo1, lo1 >> 16};
        const uint32_t hi = r.shi >> (8 * h);
        float t = 0.f;
#pragma unroll
        for (int p = 0; p < 4; p++) {
            const uint32_t top = (hi >> (16 * (p & 1) + 2 * (2 * n + (p >> 1)))) & 3u;
            const int sc = (int)((lo[p] & 15u) | (top << 4)) - 32;
            // sum (c - 4) x over the sub-block, exact power-of-two scalings
            const float cx = fmaf(A[p], kTwo24 / (float)(1 << (p < 3 ? 2 * p : 4)),
                                  -4.f * sums[sbase + 2 * p]);
            t = fmaf((float)sc, cx, t);
        }
        acc = fmaf(half_bits_to_float(r.d), t, acc);
    }
};

// ---------------------------------------------------------------------------
// 32-weight nibble formats, one block per unit (FlareLLM page, section
// "量化技术的全面支持": the standard 4- and 5-bit quantisations).  Code byte l
// (0..15) holds weight l in its low nibble and weight l + 16 in its high
// nibble; the 5-bit formats add bit i of a little-endian 32-bit word as the
// fifth bit of weight i.  w = d * (q - kOff) (Q4_0: 8, Q5_0: 16) or
// w = d * q + m (Q4_1, Q5_1, kMin); both are applied once per block through
// the block's activation sum.  kHigh: byte offset of the fifth-bit word (0:
// none); kCodes: byte offset of the 16 code bytes.
// ---------------------------------------------------------------------------
template <int kBytes, bool kMin, int kHigh, int kCodes, int kOff>
struct Nib32 {
    static constexpr int kBlockWeights = 32;
    static constexpr int kBlockBytes = kBytes;
    static constexpr int kUnitWeights = 32;
    static constexpr int kSumGroup = 32;
    static constexpr int kPadEvery = 32;
    static constexpr int kHighOff = kHigh, kCodesOff = kCodes;
    static constexpr bool kHasMin = kMin;
    struct Regs {
        uint4 q;
        uint32_t hdr;  // d (and m in the high half)
        uint32_t hb;   // fifth bits
    };
    __device__ static __forceinline__ uint32_t unit_offset(int u) { return (uint32_t)u * kBytes; }
    __device__ static __forceinline__ Regs load(const BufSrc &src, uint32_t off, int) {
        Regs r;
        r.hdr = kMin ? src.ld4(off) : src.ld2(off);
        r.hb = kHigh ? src.ld4(off + kHigh) : 0u;
        r.q = src.ld16(off + kCodes);
        return r;
    }
    // 36 floats per unit in LDS: 32 activations and 4 pad
    __device__ static __forceinline__ void load_x(const float *xs, int u, float *xv) {
        const float4 *p = reinterpret_cast<const float4 *>(xs + 36 * u);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float4 v = p[i];
            xv[4 * i] = v.x;
            xv[4 * i + 1] = v.y;
            xv[4 * i + 2] = v.z;
            xv[4 * i + 3] = v.w;
        }
    }
    // Bits 0..3 of t moved to bit 4 of bytes 0..3 (the multiply places bit
    // k at bit 8k without carries).
    __device__ static __forceinline__ uint32_t fifth_bits(uint32_t t) {
        return (((t & 15u) * 0x00204081u) & 0x01010101u) << 4;
    }
    // One block: code dwords qw, header hdr (d, and m in the high half),
    // fifth bits hb, its 32 activations xv and their sum.
    __device__ static __forceinline__ void block(const uint32_t (&qw)[4], uint32_t hdr, uint32_t hb,
                                                 const float *xv, float xsum, float &acc) {
        float lo0 = 0.f, lo1 = 0.f, hi0 = 0.f, hi1 = 0.f;
        if constexpr (!kHigh) {
            // four-bit codes: each dword masked in place (bytes 0 and 2) and
            // shifted by 8 (bytes 1 and 3), as in the Q4_K dot; the high
            // nibbles come out as 16 q
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t w = qw[i], w8 = qw[i] >> 8;
                const f16x2_t a02 = as_f16x2(w & 0x000F000Fu), a13 = as_f16x2(w8 & 0x000F000Fu);
                const f16x2_t b02 = as_f16x2(w & 0x00F000F0u), b13 = as_f16x2(w8 & 0x00F000F0u);
                lo0 = fmaf((float)a02.x, xv[4 * i + 0], lo0);
                lo1 = fmaf((float)a02.y, xv[4 * i + 2], lo1);
                lo0 = fmaf((float)a13.x, xv[4 * i + 1], lo0);
                lo1 = fmaf((float)a13.y, xv[4 * i + 3], lo1);
                hi0 = fmaf((float)b02.x, xv[16 + 4 * i + 0], hi0);
                hi1 = fmaf((float)b02.y, xv[16 + 4 * i + 2], hi1);
                hi0 = fmaf((float)b13.x, xv[16 + 4 * i + 1], hi0);
                hi1 = fmaf((float)b13.y, xv[16 + 4 * i + 3], hi1);
            }
            hi0 = (hi0 + hi1) * 0.0625f;  // exact: a power of two
            hi1 = 0.f;
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                // weights 4i .. 4i+3 and 16+4i .. 16+4i+3, with their fifth bits
                const uint32_t a = (qw[i] & 0x0F0F0F0Fu) | fifth_bits(hb >> (4 * i));
                const uint32_t b = ((qw[i] >> 4) & 0x0F0F0F0Fu) | fifth_bits(hb >> (16 + 4 * i));
                const f16x2_t a01 = as_f16x2(bytes01_to_halves(a)), a23 = as_f16x2(bytes23_to_halves(a));
                const f16x2_t b01 = as_f16x2(bytes01_to_halves(b)), b23 = as_f16x2(bytes23_to_halves(b));
                lo0 = fmaf((float)a01.x, xv[4 * i + 0], lo0);
                lo1 = fmaf((float)a01.y, xv[4 * i + 1], lo1);
                lo0 = fmaf((float)a23.x, xv[4 * i + 2], lo0);
                lo1 = fmaf((float)a23.y, xv[4 * i + 3], lo1);
                hi0 = fmaf((float)b01.x, xv[16 + 4 * i + 0], hi0);
                hi1 = fmaf((float)b01.y, xv[16 + 4 * i + 1], hi1);
                hi0 = fmaf((float)b23.x, xv[16 + 4 * i + 2], hi0);
                hi1 = fmaf((float)b23.y, xv[16 + 4 * i + 3], hi1);
            }
        }
        const float qx = ((lo0 + lo1) + (hi0 + hi1)) * kTwo24;  // sum q x, exact scaling
        const float d = half_bits_to_float(hdr);
        if constexpr (kMin) {
            acc = fmaf(d, qx, fmaf(half_bits_to_float(hdr >> 16), xsum, acc));
        } else {
            acc = fmaf(d, fmaf(-(float)kOff, xsum, qx), acc);
        }
    }
    __device__ static __forceinline__ void dot(const Regs &r, const float *xv, const float *sums,
                                               int u, float &acc) {
        const uint32_t qw[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
        block(qw, r.hdr, r.hb, xv, sums[u], acc);
    }
};
using Q40 = Nib32<18, false, 0, 2, 8>;
using Q41 = Nib32<20, true, 0, 4, 0>;
using Q50 = Nib32<22, false, 2, 6, 16>;
using Q51 = Nib32<24, true, 4, 8, 0>;

// ---------------------------------------------------------------------------
// Q4_0 and Q5_0, two blocks per unit (rows with an even number of blocks):
// their 18- and 22-byte blocks leave one-block loads only 2-byte aligned,
// while two blocks (36 and 44 bytes) start 4-byte aligned.  Block 1's
// fields then sit on whole dwords; block 0's are the dwords funnel-shifted
// by 16 bits.  Each block is computed exactly as in the one-block unit.
// ---------------------------------------------------------------------------
template <class B>
struct Nib32x2 {
    static constexpr int kBlockWeights = 32;
    static constexpr int kBlockBytes = B::kBlockBytes;
    static constexpr int kUnitWeights = 64;
    static constexpr int kSumGroup = 32;
    static constexpr int kPadEvery = 64;
    static constexpr int kHigh = B::kHighOff, kCodes = B::kCodesOff;
    static_assert(kBlockBytes % 4 == 2 && kCodes % 4 == 2 && (kHigh == 0 || kHigh % 4 == 2) && !B::kHasMin,
                  "2-byte-aligned blocks without a min field");
    static_assert(2 * kBlockBytes == 36 || 2 * kBlockBytes == 44, "Q4_0 or Q5_0");
    struct Regs {
        uint4 a, b;  // unit dwords 0 .. 7
        uint4 c;     // dwords 7 .. 10 (Q5_0), or dword 8 in .y (Q4_0)
    };
    __device__ static __forceinline__ uint32_t unit_offset(int u) {
        return (uint32_t)u * (2 * kBlockBytes);
    }
    // Every load stays inside the unit: Q5_0's last 16 bytes start at byte
    // 28, overlapping the second load by one dword.
    __device__ static __forceinline__ Regs load(const BufSrc &src, uint32_t off, int) {
        Regs r;
        r.a = src.ld16(off);
        r.b = src.ld16(off + 16);
        if constexpr (2 * kBlockBytes == 44) {
            r.c = src.ld16(off + 28);
        } else {
            r.c = make_uint4(0u, src.ld4(off + 32), 0u, 0u);
        }
        return r;
    }
    __device__ static __forceinline__ void load_x(const float *xs, int u, float *xv) {
        Q4K::load_x(xs, u, xv);
    }
    __device__ static __forceinline__ void dot(const Regs &r, const float *xv, const float *sums,
                                               int u, float &acc) {
        const uint32_t D[11] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y,
                                r.b.z, r.b.w, r.c.y, r.c.z, r.c.w};
        // block 0: fields at bytes 0 (d), kHigh, kCodes
        constexpr int c0 = kCodes / 4;  // codes start 2 bytes into D[c0]
        const uint32_t q0[4] = {__builtin_amdgcn_alignbit(D[c0 + 1], D[c0], 16),
                                __builtin_amdgcn_alignbit(D[c0 + 2], D[c0 + 1], 16),
                                __builtin_amdgcn_alignbit(D[c0 + 3], D[c0 + 2], 16),
                                __builtin_amdgcn_alignbit(D[c0 + 4], D[c0 + 3], 16)};
        const uint32_t hb0 = kHigh ? __builtin_amdgcn_alignbit(D[kHigh / 4 + 1], D[kHigh / 4], 16) : 0u;
        B::block(q0, D[0], hb0, xv, sums[2 * u], acc);
        // block 1: fields at kBlockBytes (d, the high half of a dword) and
        // kBlockBytes + kHigh / kCodes (whole dwords)
        constexpr int c1 = (kBlockBytes + kCodes) / 4;
        const uint32_t q1[4] = {D[c1], D[c1 + 1], D[c1 + 2], D[c1 + 3]};
        const uint32_t hb1 = kHigh ? D[(kBlockBytes + kHigh) / 4] : 0u;
        B::block(q1, D[kBlockBytes / 4] >> 16, hb1, xv + 32, sums[2 * u + 1], acc);
    }
};
using Q40x2 = Nib32x2<Q40>;
using Q50x2 = Nib32x2<Q50>;

// ---------------------------------------------------------------------------
// Q4_1 and Q5_1, two blocks per unit (rows with an even number of blocks):
// their 20- and 24-byte blocks are 4-byte aligned, so every field of both
// blocks sits on whole dwords (d and m in one dword, then Q5_1's fifth bits,
// then the 16 code bytes).  With 64 weights per unit a 4096-weight row is one
// unit step of 64 lanes, which keeps x in registers.  Each block is computed
// exactly as in the one-block unit.
// ---------------------------------------------------------------------------
template <class B>
struct Nib32x2m {
    static constexpr int kBlockWeights = 32;
    static constexpr int kBlockBytes = B::kBlockBytes;
    static constexpr int kUnitWeights = 64;
    static constexpr int kSumGroup = 32;
    static constexpr int kPadEvery = 64;
    static constexpr int kHigh = B::kHighOff, kCodes = B::kCodesOff;
    static_assert(kBlockBytes % 4 == 0 && kCodes % 4 == 0 && kHigh % 4 == 0 && B::kHasMin,
                  "4-byte-aligned blocks with a min field");
    static_assert(2 * kBlockBytes == 40 || 2 * kBlockBytes == 48, "Q4_1 or Q5_1");
    struct Regs {
        uint4 a, b, c;  // unit dwords 0 .. 11 (Q5_1); Q4_1: c holds dwords 6 .. 9
    };
    __device__ static __forceinline__ uint32_t unit_offset(int u) {
        return (uint32_t)u * (2 * kBlockBytes);
    }
    // Every load stays inside the unit: Q4_1's last 16 bytes start at byte
    // 24, overlapping the second load by two dwords.
    __device__ static __forceinline__ Regs load(const BufSrc &src, uint32_t off, int) {
        Regs r;
        r.a = src.ld16(off);
        r.b = src.ld16(off + 16);
        r.c = src.ld16(off + (2 * kBlockBytes == 48 ? 32 : 24));
        return r;
    }
    __device__ static __forceinline__ void load_x(const float *xs, int u, float *xv) {
        Q4K::load_x(xs, u, xv);
    }
    __device__ static __forceinline__ void dot(const Regs &r, const float *xv, const float *sums,
                                               int u, float &acc) {
        // D[i] is dword i of the unit
        uint32_t D[12];
        D[0] = r.a.x; D[1] = r.a.y; D[2] = r.a.z; D[3] = r.a.w;
        D[4] = r.b.x; D[5] = r.b.y; D[6] = r.b.z; D[7] = r.b.w;
        if constexpr (2 * kBlockBytes == 48) {
            D[8] = r.c.x; D[9] = r.c.y; D[10] = r.c.z; D[11] = r.c.w;
        } else {
            D[8] = r.c.z; D[9] = r.c.w; D[10] = 0u; D[11] = 0u;
        }
        constexpr int c0 = kCodes / 4, c1 = (kBlockBytes + kCodes) / 4;
        const uint32_t q0[4] = {D[c0], D[c0 + 1], D[c0 + 2], D[c0 + 3]};
        const uint32_t q1[4] = {D[c1], D[c1 + 1], D[c1 + 2], D[c1 + 3]};
        const uint32_t hb0 = kHigh ? D[kHigh / 4] : 0u;
        const uint32_t hb1 = kHigh ? D[(kBlockBytes + kHigh) / 4] : 0u;
        B::block(q0, D[0], hb0, xv, sums[2 * u], acc);
        B::block(q1, D[kBlockBytes / 4], hb1, xv + 32, sums[2 * u + 1], acc);
    }
};
using Q41x2 = Nib32x2m<Q41>;
using Q51x2 = Nib32x2m<Q51>;

// ---------------------------------------------------------------------------
// Q8_1 as weights: Q8_0 plus an fp16 field s (the scaled code sum, meant for
// activations, not used here); one 36-byte block per unit.
// ---------------------------------------------------------------------------
struct Q81x1 {
    static constexpr int kBlockWeights = 32;
    static constexpr int kBlockBytes = 36;
    static constexpr int kUnitWeights = 32;
    static constexpr int kSumGroup = 0;
    static constexpr int kPadEvery = 32;
    struct Regs {
        uint4 a, b;
        uint32_t c;
    };
    __device__ static __forceinline__ uint32_t unit_offset(int u) { return (uint32_t)u * 36; }
    __device__ static __forceinline__ Regs load(const BufSrc &src, uint32_t off, int) {
        Regs r;
        r.c = src.ld4(off);
        r.a = src.ld16(off + 4);
        r.b = src.ld16(off + 20);
        return r;
    }
    __device__ static __forceinline__ void load_x(const float *xs, int u, float *xv) {
        Q80x1::load_x(xs, u, xv);
    }
    __device__ static __forceinline__ void dot(const Regs &r, const float *xv, const float *sums,
                                               int u, float &acc) {
        Q80x1::Regs q;
        q.a = r.a;
        q.b = r.b;
        q.c = r.c;  // d in the low half; the sum field is ignored
        Q80x1::dot(q, xv, sums, u, acc);
    }
};

}  // namespace qmv
