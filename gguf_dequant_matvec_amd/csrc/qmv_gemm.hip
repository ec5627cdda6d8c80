// Placeholder until the small-batch MFMA kernels land.
#include "qmv_internal.h"

namespace qmv {

hipError_t launch_gemm_n(int, const uint8_t *, int64_t, int64_t, int32_t, const float *, float *,
                         hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace qmv
