// One token of the gated short convolution (BebeLM page, section "门控短卷积"):
// in_proj with the gates, the causal depthwise convolution and its state
// shift in one launch of the row-streaming kernel, then out_proj.
#include "qmv_launch.h"

namespace qmv {

hipError_t launch_short_conv(int in_t, const uint8_t *in_proj, int64_t D, int64_t H,
                             const float *h, const float *w_conv, float *state, int out_t,
                             const uint8_t *out_proj, float *out, float *y, hipStream_t s) {
    RowsParams p{};
    p.W = in_proj;
    p.M = (int32_t)D;  // channels; in_proj has 3D rows
    p.K = (int32_t)H;
    p.row_bytes = (int64_t)row_bytes_of(in_t, H);
    p.x = h;
    p.seg.n = 1;
    p.seg.start[0] = 0;
    p.seg.start[1] = (int32_t)D;
    p.seg.y[0] = y;
    p.conv_w = w_conv;
    p.conv_state = state;
    hipError_t e = launch_fmt<kModeShortConv>(in_t, p, s, nullptr);
    if (e != hipSuccess) return e;
    SegTable seg{};
    seg.n = 1;
    seg.start[0] = 0;
    seg.start[1] = (int32_t)H;
    seg.y[0] = out;
    return launch_rows_store(out_t, out_proj, H, D, y, seg, s);
}

}  // namespace qmv
