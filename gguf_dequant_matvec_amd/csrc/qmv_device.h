// Device helpers shared by the gfx950 kernels of libqmv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {

constexpr int kWave = 64;          // CDNA wavefront
constexpr int kBlockThreads = 256;  // 4 waves per workgroup
constexpr int kWideBlockThreads = 512;  // 8 waves: one workgroup per CU (long rows)
constexpr int kMaxBlockThreads = 512;

typedef float f32x2 __attribute__((ext_vector_type(2)));

// binary16 bits (low 16 bits of h) -> f32; exact, subnormals kept.
__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
}

// Loads from any byte address (gfx950 runs with unaligned global access
// enabled; each compiles to one global_load_dword{,x2,x4}).  The weight
// streams use ordinary (temporal) loads: a 128-byte line is touched by several
// lanes' loads of one block, and non-temporal loads, which skip that reuse,
// measured about 20% slower for these kernels on MI355X.
__device__ __forceinline__ uint4 load16(const uint8_t *p) {
    uint4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}
__device__ __forceinline__ uint2 load8(const uint8_t *p) {
    uint2 v;
    __builtin_memcpy(&v, p, 8);
    return v;
}
__device__ __forceinline__ uint32_t load4(const uint8_t *p) {
    uint32_t v;
    __builtin_memcpy(&v, p, 4);
    return v;
}
__device__ __forceinline__ uint32_t load2(const uint8_t *p) {
    uint16_t v;
    __builtin_memcpy(&v, p, 2);
    return v;
}

// A raw buffer view of `bytes` bytes at `base` (base and size wave-uniform).
// Loads take a per-lane byte offset and, past the end, return zeros without
// touching memory (the hardware range check), so ragged tails need no clamps.
// Every weight stream goes through these: one 32-bit offset per lane instead
// of 64-bit address arithmetic per load.
struct BufSrc {
    __amdgpu_buffer_rsrc_t rsrc;
    __device__ __forceinline__ BufSrc(const uint8_t *base, uint64_t bytes) {
        const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
        rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, (int)n,
                                                 0x00020000);  // 32-bit data format (gfx9)
    }
    __device__ __forceinline__ uint4 ld16(uint32_t off) const {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
    }
    __device__ __forceinline__ uint2 ld8(uint32_t off) const {
        return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsrc, off, 0, 0));
    }
    __device__ __forceinline__ uint32_t ld4(uint32_t off) const {
        return __builtin_amdgcn_raw_buffer_load_b32(rsrc, off, 0, 0);
    }
    __device__ __forceinline__ uint32_t ld2(uint32_t off) const {
        return __builtin_amdgcn_raw_buffer_load_b16(rsrc, off, 0, 0);
    }
};

// v with its lanes permuted by a DPP control (row-local patterns; VALU only).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane 7 - i within each 8
constexpr int kDppMirror = 0x140;       // lane 15 - i within each 16
constexpr int kDppRowRor8 = 0x128;      // lane (i + 8) mod 16 within each 16
constexpr int kDppBcast15 = 0x142;      // lane 15 of row r to row r + 1
constexpr int kDppBcast31 = 0x143;      // lane 31 to rows 2 and 3

// Byte b of a dword as an f32 integer value (v_cvt_f32_ubyteN).
template <int B>
__device__ __forceinline__ float ubyte(uint32_t v) {
    return (float)((v >> (8 * B)) & 0xFFu);
}
// Signed byte b of a dword as f32.
template <int B>
__device__ __forceinline__ float sbyte(uint32_t v) {
    return (float)(int32_t)(int8_t)((v >> (8 * B)) & 0xFFu);
}

// Codes as f16 subnormals.  A 16-bit half whose bits 10..15 are zero is the
// f16 subnormal (bits) * 2^-24, exactly; converting it to f32 is exact, and
// the compiler folds that conversion into the multiply-add (v_fma_mix_f32
// reads an f16 half of a register as one operand), so one instruction both
// converts a code and accumulates its product with an f32 activation.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
constexpr float kTwo24 = 16777216.0f;  // 2^24: undoes the subnormal scale

__device__ __forceinline__ f16x2_t as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2_t, v); }
// Bytes 0 and 1 (resp. 2 and 3) of v moved to the low byte of each half.
__device__ __forceinline__ uint32_t bytes01_to_halves(uint32_t v) {
    return __builtin_amdgcn_perm(0u, v, 0x0c010c00u);
}
__device__ __forceinline__ uint32_t bytes23_to_halves(uint32_t v) {
    return __builtin_amdgcn_perm(0u, v, 0x0c030c02u);
}

// Sum over groups of G consecutive lanes (G a power of two, 4..64), with DPP
// moves only (no LDS round trips).  The total is exact in lane G - 1 of each
// group (the group's "owner"); for G <= 16 every lane of the group has it.
// The order of the additions is fixed, so the result depends only on the
// lane values.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "lane group");
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    if (G >= 8) v += dpp_f32<kDppHalfMirror>(v);
    if (G >= 16) v += dpp_f32<kDppMirror>(v);
    if (G >= 32) {
        // rows 1 and 3 add the total of rows 0 and 2
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), kDppBcast15, 0xA, 0xF, false));
    }
    if (G == 64) {
        // row 3 adds lane 31 (rows 0 + 1)
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), kDppBcast31, 0x8, 0xF, false));
    }
    return v;
}

// Order-preserving map of an f32 to u32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_key(float v) {
    uint32_t b = __builtin_bit_cast(uint32_t, v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
    uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __builtin_bit_cast(float, b);
}

}  // namespace qmv
