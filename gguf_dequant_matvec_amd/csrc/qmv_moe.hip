// Sigmoid-routed top-k MoE FFN for one token (BebeLM page, section "核心算子",
// MoE FFN), as three launches on the caller's stream and no host round trip:
//   1. router: logits r_e = R[e, :] . x in f32, one workgroup per expert;
//   2. gate/up: every workgroup derives the selection (sigmoid, biased top-k,
//      renormalised weights) from the logits, then streams the selected
//      experts' gate and up rows, each gate row with its up row, and writes
//      g, u and h = silu(g) * u into the workspace;
//   3. down: x' = concat_s(w_s * h_s) and row i = concat_s(D_s[i]) give
//      y[i] = sum_s w_s D_s[i] . h_s in one fixed-order row sum.
// Workspace layout (bytes): [0, 256) f32 logits[E]; [256, ...) f32
// gu[k][2I] (gate rows then up rows per slot); then f32 h[k][I].
#include "qmv_launch.h"

namespace qmv {

namespace {

__global__ __launch_bounds__(256) void router_logits(const float *__restrict__ R,
                                                     const float *__restrict__ x, int H,
                                                     float *logits) {
    const int e = blockIdx.x;
    const float *row = R + (int64_t)e * H;
    float acc = 0.f;
    for (int i = threadIdx.x * 4; i < H; i += 256 * 4) {
        // x and the router rows need only 4-byte alignment (unaligned
        // 16-byte global loads are enabled on this device)
        const float4 r = __builtin_bit_cast(float4, load16(reinterpret_cast<const uint8_t *>(row + i)));
        const float4 v = __builtin_bit_cast(float4, load16(reinterpret_cast<const uint8_t *>(x + i)));
        acc = fmaf(r.x, v.x, acc);
        acc = fmaf(r.y, v.y, acc);
        acc = fmaf(r.z, v.z, acc);
        acc = fmaf(r.w, v.w, acc);
    }
    acc = group_sum<64>(acc);  // wave total in lane 63
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 63) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) logits[e] = (red[0] + red[1]) + (red[2] + red[3]);
}

}  // namespace

hipError_t launch_moe(const float *x, int64_t H, const float *router, const float *bias,
                      int32_t E, int32_t k, int gu_t, const uint8_t *gate_up, int dn_t,
                      const uint8_t *down, int64_t I, float *y, int32_t *topk_idx,
                      float *topk_w, uint8_t *ws, hipStream_t s) {
    float *logits = reinterpret_cast<float *>(ws);
    float *gu = reinterpret_cast<float *>(ws + 256);
    float *h = gu + (int64_t)k * 2 * I;

    hipError_t e = launch_aux(router_logits, dim3(E), dim3(256), 0, s, router, x, (int)H, logits);
    if (e != hipSuccess) return e;

    MoeArgs m{};
    m.logits = logits;
    m.bias = bias;
    m.E = E;
    m.k = k;
    m.topk_idx = topk_idx;
    m.topk_w = topk_w;
    m.h = h;
    m.I = (int32_t)I;

    RowsParams pg{};
    pg.W = gate_up;
    pg.M = (int32_t)(k * I);  // row pairs (gate row j, up row j)
    pg.K = (int32_t)H;
    pg.row_bytes = (int64_t)row_bytes_of(gu_t, H);
    pg.x = x;
    pg.seg.n = 1;
    pg.seg.start[0] = 0;
    pg.seg.start[1] = pg.M;
    pg.seg.y[0] = gu;
    pg.moe = m;
    pg.moe.mat_bytes = 2 * I * pg.row_bytes;
    pg.moe.rows_per_mat = (int32_t)(2 * I);
    e = launch_fmt<kModeMoeGateUp>(gu_t, pg, s, nullptr);
    if (e != hipSuccess) return e;

    RowsParams pd{};
    pd.W = down;
    pd.M = (int32_t)H;
    pd.K = (int32_t)(k * I);
    pd.row_bytes = (int64_t)row_bytes_of(dn_t, I);
    pd.x = nullptr;
    pd.seg.n = 1;
    pd.seg.start[0] = 0;
    pd.seg.start[1] = pd.M;
    pd.seg.y[0] = y;
    pd.moe = m;
    pd.moe.mat_bytes = H * pd.row_bytes;
    return launch_fmt<kModeMoeDown>(dn_t, pd, s, nullptr);
}

}  // namespace qmv
