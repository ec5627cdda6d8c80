// Placeholder until the MoE kernels land.
#include "qmv_internal.h"

namespace qmv {

hipError_t launch_moe(const float *, int64_t, const float *, const float *, int32_t, int32_t,
                      int, const uint8_t *, int, const uint8_t *, int64_t, float *, int32_t *,
                      float *, uint8_t *, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace qmv
