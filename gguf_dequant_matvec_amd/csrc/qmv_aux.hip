// Dequantisation export, weight quantisation and the HBM read probe.
#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {

namespace {

// ---------------------------------------------------------------------------
// Dequantise: thread t writes weights [16t, 16t + 16) of the flat matrix.
// Values are the exact block decodings (Q4_K: (d*sc)*q - dmin*m with one
// rounding; the others exact), the surface the matvecs are defined on.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store16(float *out, const float *v) {
    float4 *o = reinterpret_cast<float4 *>(out);
#pragma unroll
    for (int i = 0; i < 4; i++) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

__global__ void dequant_q8_0(const uint8_t *W, int64_t ngroups, float *out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= ngroups) return;
    const uint8_t *blk = W + (t >> 1) * 34;
    const int half = (int)(t & 1);
    const float d = half_bits_to_float(load2(blk));
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] = d * (float)(int8_t)blk[2 + 16 * half + i];
    store16(out + t * 16, v);
}

__global__ void dequant_q4_k(const uint8_t *W, int64_t ngroups, float *out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= ngroups) return;
    const uint8_t *blk = W + (t >> 4) * 144;
    const int i0 = 16 * (int)(t & 15);
    const int j = i0 / 32, c = i0 / 64, hi = (i0 % 64) / 32, l0 = i0 % 32;
    const uint8_t *S = blk + 4;
    int sc, m;
    if (j < 4) {
        sc = S[j] & 63;
        m = S[j + 4] & 63;
    } else {
        sc = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);
        m = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
    }
    const float s = half_bits_to_float(load2(blk)) * (float)sc;
    const float o = half_bits_to_float(load2(blk + 2)) * (float)m;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const uint8_t byte = blk[16 + 32 * c + l0 + i];
        const int q = hi ? (byte >> 4) : (byte & 15);
        v[i] = s * (float)q - o;
    }
    store16(out + t * 16, v);
}

__global__ void dequant_q6_k(const uint8_t *W, int64_t ngroups, float *out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= ngroups) return;
    const uint8_t *blk = W + (t >> 4) * 210;
    const int i0 = 16 * (int)(t & 15);
    const int n = i0 / 128, g = (i0 % 128) / 32, l0 = i0 % 32;
    const float s = half_bits_to_float(load2(blk + 208)) * (float)(int8_t)blk[192 + i0 / 16];
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int l = l0 + i;
        const int lo = (blk[64 * n + l + 32 * (g & 1)] >> (4 * (g >> 1))) & 15;
        const int h2 = (blk[128 + 32 * n + l] >> (2 * g)) & 3;
        v[i] = s * (float)((lo | (h2 << 4)) - 32);
    }
    store16(out + t * 16, v);
}

// Q5_K: the Q4_K decoding with a fifth code bit, bit 2c + h of high byte l.
__global__ void dequant_q5_k(const uint8_t *W, int64_t ngroups, float *out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= ngroups) return;
    const uint8_t *blk = W + (t >> 4) * 176;
    const int i0 = 16 * (int)(t & 15);
    const int j = i0 / 32, c = i0 / 64, hi = (i0 % 64) / 32, l0 = i0 % 32;
    const uint8_t *S = blk + 4;
    int sc, m;
    if (j < 4) {
        sc = S[j] & 63;
        m = S[j + 4] & 63;
    } else {
        sc = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);
        m = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
    }
    const float s = half_bits_to_float(load2(blk)) * (float)sc;
    const float o = half_bits_to_float(load2(blk + 2)) * (float)m;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int l = l0 + i;
        const int q = ((blk[48 + 32 * c + l] >> (4 * hi)) & 15) | (((blk[16 + l] >> (2 * c + hi)) & 1) << 4);
        v[i] = s * (float)q - o;
    }
    store16(out + t * 16, v);
}

// Q2_K: thread t writes sub-block j = t & 15 of block t >> 4; weight
// 16j + i sits at plane p = (j / 2) & 3 of code byte 32n + 16(j & 1) + i
// (n = j / 8).  w = (d*sc)*q - dmin*m.
__global__ void dequant_q2_k(const uint8_t *W, int64_t ngroups, float *out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= ngroups) return;
    const uint8_t *blk = W + (t >> 4) * 84;
    const int j = (int)(t & 15), n = j >> 3, p = (j >> 1) & 3, l0 = 16 * (j & 1);
    const float s = half_bits_to_float(load2(blk + 80)) * (float)(blk[j] & 15);
    const float o = half_bits_to_float(load2(blk + 82)) * (float)(blk[j] >> 4);
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int q = (blk[16 + 32 * n + l0 + i] >> (2 * p)) & 3;
        v[i] = s * (float)q - o;
    }
    store16(out + t * 16, v);
}

// Q3_K: as Q2_K for the code position; bit 4n + p of H[16(j & 1) + i] set
// keeps the code, clear lowers it by 4; 6-bit scale minus 32.  w = (d*sc)*q.
__global__ void dequant_q3_k(const uint8_t *W, int64_t ngroups, float *out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= ngroups) return;
    const uint8_t *blk = W + (t >> 4) * 110;
    const int j = (int)(t & 15), n = j >> 3, p = (j >> 1) & 3, l0 = 16 * (j & 1);
    const uint8_t *S = blk + 96;
    const int lo4 = (S[j & 7] >> (4 * (j >> 3))) & 15;
    const int top = (S[8 + (j & 3)] >> (2 * (j >> 2))) & 3;
    const float s = half_bits_to_float(load2(blk + 108)) * (float)((lo4 | (top << 4)) - 32);
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int l = l0 + i;
        const int low = (blk[32 + 32 * n + l] >> (2 * p)) & 3;
        const int q = low - (((blk[l] >> (4 * n + p)) & 1) ? 0 : 4);
        v[i] = s * (float)q;
    }
    store16(out + t * 16, v);
}

// 32-weight nibble formats: thread t writes half h = t & 1 of block t >> 1,
// i.e. the low (h = 0) or high (h = 1) nibbles of the 16 code bytes.
// w = d * (q - kOff), or d * q + m (kMin; the product is exact, so the one
// rounding is the same with or without contraction).
template <int kBytes, bool kMin, int kHigh, int kCodes, int kOff>
__global__ void dequant_nib32(const uint8_t *W, int64_t ngroups, float *out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= ngroups) return;
    const uint8_t *blk = W + (t >> 1) * kBytes;
    const int h = (int)(t & 1);
    const float d = half_bits_to_float(load2(blk));
    const float m = kMin ? half_bits_to_float(load2(blk + 2)) : 0.f;
    uint32_t H = 0;
    if (kHigh)
        H = (uint32_t)blk[kHigh] | ((uint32_t)blk[kHigh + 1] << 8) | ((uint32_t)blk[kHigh + 2] << 16) |
            ((uint32_t)blk[kHigh + 3] << 24);
    float v[16];
#pragma unroll
    for (int l = 0; l < 16; l++) {
        int q = (blk[kCodes + l] >> (4 * h)) & 15;
        if (kHigh) q |= (int)((H >> (16 * h + l)) & 1u) << 4;
        v[l] = kMin ? d * (float)q + m : d * (float)(q - kOff);
    }
    store16(out + t * 16, v);
}

__global__ void dequant_q8_1(const uint8_t *W, int64_t ngroups, float *out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= ngroups) return;
    const uint8_t *blk = W + (t >> 1) * 36;
    const int half = (int)(t & 1);
    const float d = half_bits_to_float(load2(blk));
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] = d * (float)(int8_t)blk[4 + 16 * half + i];
    store16(out + t * 16, v);
}

// ---------------------------------------------------------------------------
// Quantise: one thread per block, f32 arithmetic without contraction so the
// bytes are reproducible: Q8_0 d = max|w|/127, q = round(w * (1/d));
// Q4_K mins first (dmin = max(-min)/62, m = ceil(-min/dmin)), then scales
// (s = (max - L)/15, d = max s / 62, sc = ceil(s/d)), q = round((w - L)/(d*sc));
// Q6_K s = max|w|/31, d = max s/126, sc = ceil(s/d), q = round(w/(d*sc)).
// Rounding is half away from zero; binary16 stores round to nearest even.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t to_half_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__global__ void quantize_q8_0(const float *w, int64_t nblocks, uint8_t *out) {
#pragma clang fp contract(off)
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    const float *src = w + b * 32;
    uint8_t *dst = out + b * 34;
    float amax = 0.f;
    for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(src[i]));
    const float d = amax / 127.0f;
    const float id = d != 0.f ? 1.0f / d : 0.f;
    const uint16_t dh = to_half_bits(d);
    dst[0] = (uint8_t)(dh & 255);
    dst[1] = (uint8_t)(dh >> 8);
    for (int i = 0; i < 32; i++) {
        float v = roundf(src[i] * id);
        v = fminf(fmaxf(v, -128.f), 127.f);
        dst[2 + i] = (uint8_t)(int8_t)v;
    }
}

__global__ void quantize_q4_k(const float *w, int64_t nblocks, uint8_t *out) {
#pragma clang fp contract(off)
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    const float *src = w + b * 256;
    uint8_t *dst = out + b * 144;
    float lo[8], hi[8], L[8], s[8];
    int sc[8], m[8];
    float maxneg = 0.f, maxs = 0.f;
    for (int j = 0; j < 8; j++) {
        float mn = 0.f, mx = -__builtin_inff();
        for (int t = 0; t < 32; t++) {
            const float v = src[32 * j + t];
            mn = v < mn ? v : mn;
            mx = v > mx ? v : mx;
        }
        lo[j] = mn;
        hi[j] = mx;
        maxneg = -mn > maxneg ? -mn : maxneg;
    }
    const uint16_t dminh = to_half_bits(maxneg / 62.0f);
    const float dmin16 = half_bits_to_float(dminh);
    for (int j = 0; j < 8; j++) {
        int mj = 0;
        if (dmin16 > 0.f) {
            const float t = ceilf(-lo[j] / dmin16);
            mj = t > 63.f ? 63 : (int)t;
        }
        m[j] = mj;
        L[j] = -(dmin16 * (float)mj);
        s[j] = (hi[j] - L[j]) / 15.0f;
        maxs = s[j] > maxs ? s[j] : maxs;
    }
    const uint16_t dh = to_half_bits(maxs / 62.0f);
    const float d16 = half_bits_to_float(dh);
    for (int j = 0; j < 8; j++) {
        int sj = 0;
        if (d16 > 0.f) {
            const float t = ceilf(s[j] / d16);
            sj = t > 63.f ? 63 : (int)t;
        }
        sc[j] = sj;
    }
    dst[0] = (uint8_t)(dh & 255);
    dst[1] = (uint8_t)(dh >> 8);
    dst[2] = (uint8_t)(dminh & 255);
    dst[3] = (uint8_t)(dminh >> 8);
    for (int j = 0; j < 4; j++) {
        dst[4 + j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        dst[8 + j] = (uint8_t)((m[j] & 63) | ((m[j + 4] >> 4) << 6));
        dst[12 + j] = (uint8_t)((sc[j + 4] & 15) | ((m[j + 4] & 15) << 4));
    }
    for (int c = 0; c < 4; c++) {
        for (int l = 0; l < 32; l++) {
            int qv[2];
            for (int h = 0; h < 2; h++) {
                const int j = 2 * c + h;
                const float v = src[64 * c + 32 * h + l];
                int q = 0;
                if (sc[j] > 0) {
                    const float step = d16 * (float)sc[j];
                    float t = roundf((v - L[j]) / step);
                    t = fminf(fmaxf(t, 0.f), 15.f);
                    q = (int)t;
                }
                qv[h] = q;
            }
            dst[16 + 32 * c + l] = (uint8_t)(qv[0] | (qv[1] << 4));
        }
    }
}

__global__ void quantize_q6_k(const float *w, int64_t nblocks, uint8_t *out) {
#pragma clang fp contract(off)
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    const float *src = w + b * 256;
    uint8_t *dst = out + b * 210;
    float s[16], maxs = 0.f;
    int sc[16];
    for (int j = 0; j < 16; j++) {
        float amax = 0.f;
        for (int t = 0; t < 16; t++) amax = fmaxf(amax, fabsf(src[16 * j + t]));
        s[j] = amax / 31.0f;
        maxs = s[j] > maxs ? s[j] : maxs;
    }
    const uint16_t dh = to_half_bits(maxs / 126.0f);
    const float d16 = half_bits_to_float(dh);
    for (int j = 0; j < 16; j++) {
        int sj = 0;
        if (d16 > 0.f) {
            const float t = ceilf(s[j] / d16);
            sj = t > 127.f ? 127 : (int)t;
        }
        sc[j] = sj;
        dst[192 + j] = (uint8_t)(int8_t)sj;
    }
    dst[208] = (uint8_t)(dh & 255);
    dst[209] = (uint8_t)(dh >> 8);
    // codes u = q + 32 in 0..63, packed: low nibbles into QL, high pairs into QH
    for (int n = 0; n < 2; n++) {
        for (int l = 0; l < 32; l++) {
            int u[4];
            for (int g = 0; g < 4; g++) {
                const int i = 128 * n + 32 * g + l;
                const int j = i / 16;
                int q = 0;
                if (sc[j] > 0) {
                    const float step = d16 * (float)sc[j];
                    float t = roundf(src[i] / step);
                    t = fminf(fmaxf(t, -32.f), 31.f);
                    q = (int)t;
                }
                u[g] = q + 32;
            }
            dst[64 * n + l] = (uint8_t)((u[0] & 15) | ((u[2] & 15) << 4));
            dst[64 * n + 32 + l] = (uint8_t)((u[1] & 15) | ((u[3] & 15) << 4));
            dst[128 + 32 * n + l] =
                (uint8_t)((u[0] >> 4) | ((u[1] >> 4) << 2) | ((u[2] >> 4) << 4) | ((u[3] >> 4) << 6));
        }
    }
}

// ---------------------------------------------------------------------------
// HBM read probe: each wave streams 4 KB chunks (chunk = wave + k * waves),
// four 1 KB loads in flight, nontemporal (every line is read by one load
// only, so skipping the caches loses nothing), xor-folded into one word per
// workgroup.  Of the patterns measured on MI355X (grid-stride or contiguous
// chunks, 1-4 workgroups per compute unit, plain, nontemporal or sc1 loads)
// this one reads fastest, so it stands for the achievable ceiling.
// ---------------------------------------------------------------------------
constexpr uint32_t kProbeChunk = 4096;

__global__ __launch_bounds__(256) void probe_read(const uint8_t *buf, uint64_t bytes, uint32_t *sink) {
    const int lane = threadIdx.x & 63;
    const uint64_t nw = (uint64_t)gridDim.x * 4;
    uint32_t acc = 0;
    for (uint64_t c = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6); c * kProbeChunk < bytes; c += nw) {
        const uint64_t left = bytes - c * kProbeChunk;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(buf + c * kProbeChunk), (short)0,
            (int)(left < kProbeChunk ? left : kProbeChunk), 0x00020000);
        uint4 v[4];
#pragma unroll
        for (int j = 0; j < 4; j++)  // past the end of the buffer the loads return zeros
            v[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 r, (uint32_t)(1024 * j + 16 * lane), 0, 2 /* nt */));
#pragma unroll
        for (int j = 0; j < 4; j++) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    __shared__ uint32_t red[4];
    if (lane == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

hipError_t launch_dequant(int type, const uint8_t *W, int64_t M, int64_t K, float *out,
                          hipStream_t s) {
    const int64_t ngroups = M * K / 16;
    if ((ngroups + 255) / 256 > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)((ngroups + 255) / 256);
    switch (type) {
    case kQ80: return launch_main(dequant_q8_0, dim3(grid), dim3(256), 0, s, W, ngroups, out);
    case kQ4K: return launch_main(dequant_q4_k, dim3(grid), dim3(256), 0, s, W, ngroups, out);
    case kQ6K: return launch_main(dequant_q6_k, dim3(grid), dim3(256), 0, s, W, ngroups, out);
    case kQ5K: return launch_main(dequant_q5_k, dim3(grid), dim3(256), 0, s, W, ngroups, out);
    case kQ2K: return launch_main(dequant_q2_k, dim3(grid), dim3(256), 0, s, W, ngroups, out);
    case kQ3K: return launch_main(dequant_q3_k, dim3(grid), dim3(256), 0, s, W, ngroups, out);
    case kQ40:
        return launch_main((dequant_nib32<18, false, 0, 2, 8>), dim3(grid), dim3(256), 0, s, W, ngroups, out);
    case kQ41:
        return launch_main((dequant_nib32<20, true, 0, 4, 0>), dim3(grid), dim3(256), 0, s, W, ngroups, out);
    case kQ50:
        return launch_main((dequant_nib32<22, false, 2, 6, 16>), dim3(grid), dim3(256), 0, s, W, ngroups, out);
    case kQ51:
        return launch_main((dequant_nib32<24, true, 4, 8, 0>), dim3(grid), dim3(256), 0, s, W, ngroups, out);
    case kQ81: return launch_main(dequant_q8_1, dim3(grid), dim3(256), 0, s, W, ngroups, out);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_quantize(int type, const float *w, int64_t M, int64_t K, uint8_t *out,
                           hipStream_t s) {
    const int64_t nblocks = M * (K / block_weights_of(type));
    if ((nblocks + 127) / 128 > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)((nblocks + 127) / 128);
    switch (type) {
    case kQ80: return launch_main(quantize_q8_0, dim3(grid), dim3(128), 0, s, w, nblocks, out);
    case kQ4K: return launch_main(quantize_q4_k, dim3(grid), dim3(128), 0, s, w, nblocks, out);
    case kQ6K: return launch_main(quantize_q6_k, dim3(grid), dim3(128), 0, s, w, nblocks, out);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s) {
    int grid = device_cu_count() * 2;  // two workgroups per compute unit
    if (grid > 2048) grid = 2048;
    return launch_main(probe_read, dim3(grid), dim3(256), 0, s, (const uint8_t *)buf,
                       (uint64_t)bytes, sink);
}

}  // namespace qmv
