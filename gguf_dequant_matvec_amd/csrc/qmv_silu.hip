// Fused gate/up with the SiLU-gated product, h = silu(g) * u, as one launch
// of the row-streaming kernel (BebeLM page, section "核心算子": the gated FFN;
// FlareLLM page, section "推理层面的深度优化": gate and up fused).
#include "qmv_launch.h"

namespace qmv {

hipError_t launch_rows_silu(int type, const uint8_t *W, int64_t I, int64_t K, const float *x,
                            float *h, hipStream_t s) {
    RowsParams p{};
    p.W = W;
    p.M = (int32_t)I;  // output rows; the matrix has 2I
    p.K = (int32_t)K;
    p.row_bytes = (int64_t)row_bytes_of(type, K);
    p.x = x;
    p.seg.n = 1;
    p.seg.start[0] = 0;
    p.seg.start[1] = (int32_t)I;
    p.seg.y[0] = h;
    p.partials = nullptr;
    return launch_fmt<kModeSiluUp>(type, p, s, nullptr);
}

}  // namespace qmv
