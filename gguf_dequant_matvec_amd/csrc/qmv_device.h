// Device helpers shared by the gfx950 kernels of libqmv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {

constexpr int kWave = 64;          // CDNA wavefront
constexpr int kBlockThreads = 256;  // 4 waves per workgroup

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

// Four bytes of v, each holding a value 0..15, to f32 scaled by 2^-9.
// A byte 0000qqqq read as an OCP fp8 e4m3 code is a subnormal (q < 8) or lies
// in the first normal binade (q >= 8); both cases decode to exactly q * 2^-9,
// so one conversion instruction turns two nibbles into two floats.
__device__ __forceinline__ void nib4_to_f32_x512(uint32_t v, float &a, float &b, float &c,
                                                 float &d) {
    f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(v, false);
    f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(v, true);
    a = lo.x;
    b = lo.y;
    c = hi.x;
    d = hi.y;
}

// Sum over groups of G consecutive lanes (G a power of two <= 64); every lane
// of the group ends with the group total.  Butterfly order is fixed, so the
// result does not depend on which rows the wave processes.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
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
