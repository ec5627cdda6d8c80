// Small-batch verify: Y[n][M] = X[n][K] . dequant(W)^T for n <= 16 on the
// matrix cores (FlareLLM page, section "推理层面的深度优化": n-gram speculative
// decoding checks several drafted tokens against the same weights).
//
// Exactness plan (the result stays within the f32 matvec's 1e-5 sum|w x|):
//  - the MFMA's weight operand holds the raw integer codes, which bf16
//    represents exactly (written 0x43uu = 128 + u, the +128 folded into a
//    per-sub-block correction); the f32 scales d*sc and mins are applied to
//    the f32 MFMA result once per sub-block;
//  - X is split into bf16 hi + lo (two MFMAs into one accumulator), so the
//    only representation error is |x - hi - lo| <= 2^-18 |x|.
// Operand roles: tokens are the MFMA M side (A = X fragment), weight rows the
// N side (B = codes), so a lane's accumulators all belong to the row whose
// block header that lane loaded and the scales apply lane-locally.
//   v_mfma_f32_16x16x32_bf16 (Q4_K, Q8_0: one 32-weight sub-block / block) and
//   v_mfma_f32_16x16x16_bf16 (Q6_K: one 16-weight sub-block); lane l of wave
//   supplies A[l%16][kpl*(l/16) + t], B[kpl*(l/16) + t][l%16] and holds
//   C[4*(l/16) + i][l%16].
// Work split: a workgroup = 4 waves x 16 rows and a K-slice of KS
// super-blocks (256 weights); X for the slice is staged once in LDS in the
// operand layout.  Slices > 1 write partial sums to the workspace and a second
// kernel adds them in slice order (deterministic, no atomics).
#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTok = 16;          // MFMA M side: tokens, n padded to 16
constexpr int kMaxSlicesSB = 4;   // super-blocks per K-slice at most (LDS budget)
constexpr uint32_t kB16 = 0x43004300u;  // bf16 128.0 in both halves

struct GemmParams {
    const uint8_t *W;
    int32_t M, K, n;
    int64_t row_bytes;
    const float *X;
    float *Y;         // final output (one slice) ...
    float *partial;   // ... or [slices][kTok][M] partial sums
    int32_t ks;       // super-blocks per slice
    int32_t slices;
};

// ---------------------------------------------------------------------------
// Format policies.  kSub: weights per MFMA sub-block (= MFMA K); kNSub:
// sub-blocks per 256-weight super-block; kKpl: operand values per lane.
// slot(i): where weight i (0..255) of a super-block sits in the operand
// layout, as (sub-block j, lane group q, slot t).
// ---------------------------------------------------------------------------
struct GQ4K {
    static constexpr int kSub = 32, kNSub = 8, kKpl = 8, kBlockBytes = 144;
    struct Regs {
        uint4 hdr;
        uint2 piece[4];  // nibble bytes 32c + 8q .. +8, c = 0..3
    };
    // k-slot t of lane group q in sub-block 2c + h is nibble h of byte
    // 8q + pi(t) of chunk c, pi = (0 2 1 3 4 6 5 7): the order in which two
    // and-or operations pull nibble pairs out of a dword.
    __device__ static void slot(int i, int &j, int &q, int &t) {
        const int c = i / 64, h = (i % 64) / 32, l = i % 32;
        j = 2 * c + h;
        q = l / 8;
        const int b = l % 8;
        t = (b & 4) | ((b & 1) << 1) | ((b & 2) >> 1);
    }
    __device__ static Regs load(const uint8_t *blk, int q) {
        Regs r;
        r.hdr = load16(blk);
#pragma unroll
        for (int c = 0; c < 4; c++) r.piece[c] = load8(blk + 16 + 32 * c + 8 * q);
        return r;
    }
    __device__ static bf16x8 codes(const Regs &r, int j) {
        const uint2 p = r.piece[j >> 1];
        const int sh = (j & 1) * 4;
        uint32_t d[4];
        d[0] = ((p.x >> sh) & 0x000F000Fu) | kB16;
        d[1] = ((p.x >> (sh + 8)) & 0x000F000Fu) | kB16;
        d[2] = ((p.y >> sh) & 0x000F000Fu) | kB16;
        d[3] = ((p.y >> (sh + 8)) & 0x000F000Fu) | kB16;
        return __builtin_bit_cast(bf16x8, d);
    }
    // y += scale * C - corr * sum(x): w = d*sc*q - dmin*m and the codes are q + 128
    __device__ static void scales(const Regs &r, int j, float &scale, float &corr) {
        const uint8_t *S = reinterpret_cast<const uint8_t *>(&r.hdr) + 4;
        int sc, m;
        if (j < 4) {
            sc = S[j] & 63;
            m = S[j + 4] & 63;
        } else {
            sc = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);
            m = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
        }
        const float d = half_bits_to_float(r.hdr.x), dmin = half_bits_to_float(r.hdr.x >> 16);
        scale = d * (float)sc;
        corr = fmaf(128.0f, scale, dmin * (float)m);
    }
};

struct GQ6K {
    static constexpr int kSub = 16, kNSub = 16, kKpl = 4, kBlockBytes = 210;
    struct Regs {
        uint32_t ql[2][2][2];  // [n][g&1][hh]: QL bytes 64n + 32(g&1) + 16hh + 4q .. +4
        uint32_t qh[2][2];     // [n][hh]: QH bytes 32n + 16hh + 4q .. +4
        uint4 sc;
        uint32_t d;
    };
    // weight i = 128n + 32g + 16hh + 4q + t, sub-block j = 8n + 2g + hh
    __device__ static void slot(int i, int &j, int &q, int &t) {
        const int n = i / 128, g = (i % 128) / 32, l = i % 32, hh = l / 16;
        j = 8 * n + 2 * g + hh;
        q = (l % 16) / 4;
        t = l % 4;
    }
    __device__ static Regs load(const uint8_t *blk, int q) {
        Regs r;
#pragma unroll
        for (int n = 0; n < 2; n++)
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int hh = 0; hh < 2; hh++) r.ql[n][a][hh] = load4(blk + 64 * n + 32 * a + 16 * hh + 4 * q);
#pragma unroll
        for (int n = 0; n < 2; n++)
#pragma unroll
            for (int hh = 0; hh < 2; hh++) r.qh[n][hh] = load4(blk + 128 + 32 * n + 16 * hh + 4 * q);
        r.sc = load16(blk + 192);
        r.d = load2(blk + 208);
        return r;
    }
    __device__ static s16x4 codes(const Regs &r, int j) {
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
    __device__ static void scales(const Regs &r, int j, float &scale, float &corr) {
        const int8_t sc = reinterpret_cast<const int8_t *>(&r.sc)[j];
        scale = half_bits_to_float(r.d) * (float)sc;
        corr = 160.0f * scale;
    }
};

struct GQ80 {
    // a "super-block" is 8 consecutive Q8_0 blocks; block j is sub-block j
    static constexpr int kSub = 32, kNSub = 8, kKpl = 8, kBlockBytes = 34;
    struct Regs {
        uint2 q[8];
        uint32_t d[8];
    };
    __device__ static void slot(int i, int &j, int &q, int &t) {
        j = i / 32;
        q = (i % 32) / 8;
        t = i % 8;
    }
    // blk points at the first of the 8 blocks; nvalid of them exist
    __device__ static Regs load(const uint8_t *blk, int q, int nvalid) {
        Regs r;
#pragma unroll
        for (int b = 0; b < 8; b++) {
            const uint8_t *p = blk + 34 * (b < nvalid ? b : nvalid - 1);
            r.d[b] = load2(p);
            r.q[b] = load8(p + 2 + 8 * q);
        }
        return r;
    }
    __device__ static bf16x8 codes(const Regs &r, int j) {
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
    __device__ static void scales(const Regs &r, int j, float &scale, float &corr) {
        scale = half_bits_to_float(r.d[j]);
        corr = 0.f;
    }
};

template <class F>
__device__ __forceinline__ typename F::Regs load_sb(const uint8_t *row, int sb, int q, int nblocks) {
    if constexpr (std::is_same<F, GQ80>::value) {
        const int b0 = sb * 8;
        return F::load(row + (int64_t)b0 * 34, q, nblocks - b0 < 8 ? nblocks - b0 : 8);
    } else {
        return F::load(row + (int64_t)sb * F::kBlockBytes, q);
    }
}

template <class F>
__device__ __forceinline__ f32x4 mfma(const typename std::conditional<F::kKpl == 8, bf16x8, s16x4>::type &a,
                                      const typename std::conditional<F::kKpl == 8, bf16x8, s16x4>::type &b,
                                      f32x4 c) {
    if constexpr (F::kKpl == 8)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <class F>
__global__ __launch_bounds__(256) void gemm_n_kernel(GemmParams p) {
    using Frag = typename std::conditional<F::kKpl == 8, bf16x8, s16x4>::type;
    // LDS: X fragments for the slice, hi and lo, [sb][j][q][token] x kKpl
    // bf16, then the per-(sb, j, token) sums of hi + lo.
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int frag_vals = p.ks * F::kNSub * 4 * kTok * F::kKpl;
    __bf16 *xhi = reinterpret_cast<__bf16 *>(smem);
    __bf16 *xlo = xhi + frag_vals;
    float *xs = reinterpret_cast<float *>(xlo + frag_vals);

    const int row_blocks = (p.M + 63) / 64;
    const int rb = blockIdx.x % row_blocks;
    const int slice = blockIdx.x / row_blocks;
    const int k0 = slice * p.ks * 256;  // first weight of the slice
    const int nw = p.ks * 256;          // weights of the slice (some may lie past K)

    // --- stage X[0..16)[k0 .. k0 + nw) ------------------------------------
    for (int idx = threadIdx.x; idx < kTok * nw; idx += 256) {
        const int t = idx / nw, kk = idx - t * nw, k = k0 + kk;
        const float v = (t < p.n && k < p.K) ? p.X[(int64_t)t * p.K + k] : 0.f;
        const __bf16 hi = (__bf16)v;
        const __bf16 lo = (__bf16)(v - (float)hi);
        const int sb = kk / 256;
        int j, q, s;
        F::slot(kk % 256, j, q, s);
        const int pos = (((sb * F::kNSub + j) * 4 + q) * kTok + t) * F::kKpl + s;
        xhi[pos] = hi;
        xlo[pos] = lo;
        // sum of the represented value over the sub-block: kSub consecutive
        // indices of one token, i.e. kSub consecutive threads
        float sum = (float)hi + (float)lo;
#pragma unroll
        for (int o = 1; o < F::kSub; o <<= 1) sum += __shfl_xor(sum, o, 64);
        if ((kk % F::kSub) == 0) xs[(sb * F::kNSub + j) * kTok + t] = sum;
    }
    __syncthreads();

    // --- stream this wave's 16 rows over the slice -------------------------
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int row = rb * 64 + wave * 16 + r;
    const int rowc = row < p.M ? row : p.M - 1;
    const uint8_t *wrow = p.W + (int64_t)rowc * p.row_bytes;
    const int nblocks = p.K / (std::is_same<F, GQ80>::value ? 32 : 256);
    const int sb_total = (p.K + 255) / 256;
    const int sb0 = slice * p.ks;
    const int sb1 = (sb0 + p.ks < sb_total) ? sb0 + p.ks : sb_total;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (sb0 < sb1) {
        typename F::Regs cur = load_sb<F>(wrow, sb0, q, nblocks);
        for (int sb = sb0; sb < sb1; sb++) {
            // prefetch the next super-block (repeats the last one at the end)
            const typename F::Regs nxt = load_sb<F>(wrow, sb + 1 < sb1 ? sb + 1 : sb, q, nblocks);
            const int lsb = sb - sb0;
            const int nsub = std::is_same<F, GQ80>::value
                                 ? ((nblocks - sb * 8) < 8 ? (nblocks - sb * 8) : 8)
                                 : F::kNSub;
#pragma unroll
            for (int j = 0; j < F::kNSub; j++) {
                if (j >= nsub) break;
                const int base = ((lsb * F::kNSub + j) * 4 + q) * kTok + r;
                const Frag ah = *reinterpret_cast<const Frag *>(xhi + base * F::kKpl);
                const Frag al = *reinterpret_cast<const Frag *>(xlo + base * F::kKpl);
                const auto b = F::codes(cur, j);
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
                c = mfma<F>(ah, b, c);
                c = mfma<F>(al, b, c);
                float scale, corr;
                F::scales(cur, j, scale, corr);
                const float4 sx = *reinterpret_cast<const float4 *>(xs + (lsb * F::kNSub + j) * kTok + 4 * q);
                acc[0] = fmaf(scale, c[0], fmaf(-corr, sx.x, acc[0]));
                acc[1] = fmaf(scale, c[1], fmaf(-corr, sx.y, acc[1]));
                acc[2] = fmaf(scale, c[2], fmaf(-corr, sx.z, acc[2]));
                acc[3] = fmaf(scale, c[3], fmaf(-corr, sx.w, acc[3]));
            }
            cur = nxt;
        }
    }

    // --- tokens 4q .. 4q+3 of this lane's row --------------------------------
    if (row < p.M) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int t = 4 * q + i;
            if (p.slices == 1) {
                if (t < p.n) p.Y[(int64_t)t * p.M + row] = acc[i];
            } else {
                p.partial[((int64_t)slice * kTok + t) * p.M + row] = acc[i];
            }
        }
    }
}

// Y[t][i] = sum over slices, in slice order.
__global__ __launch_bounds__(256) void gemm_n_reduce(const float *partial, int slices, int M,
                                                     int n, float *Y) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)n * M) return;
    const int t = (int)(idx / M), i = (int)(idx - (int64_t)t * M);
    float s = 0.f;
    for (int sl = 0; sl < slices; sl++) s += partial[((int64_t)sl * kTok + t) * M + i];
    Y[idx] = s;
}

// Slicing of K: enough workgroups for the chip (about 512), at most
// kMaxSlicesSB super-blocks of X staged per workgroup.
void plan(int64_t M, int64_t K, int &ks, int &slices) {
    const int sb_total = (int)((K + 255) / 256);
    const int row_blocks = (int)((M + 63) / 64);
    int want = (512 + row_blocks - 1) / row_blocks;
    if (want < 1) want = 1;
    if (want > sb_total) want = sb_total;
    ks = (sb_total + want - 1) / want;
    if (ks > kMaxSlicesSB) ks = kMaxSlicesSB;
    slices = (sb_total + ks - 1) / ks;
}

template <class F>
hipError_t launch_typed(const GemmParams &p, hipStream_t s) {
    const int row_blocks = (p.M + 63) / 64;
    const size_t frag_vals = (size_t)p.ks * F::kNSub * 4 * kTok * F::kKpl;
    const size_t lds = frag_vals * 2 * 2 + (size_t)p.ks * F::kNSub * kTok * 4;
    hipError_t e = ensure_lds((const void *)gemm_n_kernel<F>, lds);
    if (e != hipSuccess) return e;
    hipError_t e2 = launch_main(gemm_n_kernel<F>, dim3((unsigned)(row_blocks * p.slices)), dim3(256),
                                lds, s, p);
    if (e2 != hipSuccess || p.slices == 1) return e2;
    const int64_t total = (int64_t)p.n * p.M;
    hipLaunchKernelGGL(gemm_n_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       p.partial, p.slices, p.M, p.n, p.Y);
    return hipGetLastError();
}

}  // namespace

size_t gemm_n_workspace(int64_t M, int64_t K) {
    int ks, slices;
    plan(M, K, ks, slices);
    return slices > 1 ? (size_t)slices * kTok * (size_t)M * sizeof(float) : 0;
}

hipError_t launch_gemm_n(int type, const uint8_t *W, int64_t M, int64_t K, int32_t n,
                         const float *X, float *Y, void *ws, hipStream_t s) {
    GemmParams p{};
    p.W = W;
    p.M = (int32_t)M;
    p.K = (int32_t)K;
    p.n = n;
    p.row_bytes = (int64_t)row_bytes_of(type, K);
    p.X = X;
    p.Y = Y;
    p.partial = reinterpret_cast<float *>(ws);
    plan(M, K, p.ks, p.slices);
    switch (type) {
    case kQ4K: return launch_typed<GQ4K>(p, s);
    case kQ6K: return launch_typed<GQ6K>(p, s);
    case kQ80: return launch_typed<GQ80>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qmv
