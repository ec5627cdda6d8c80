// Explicit instantiation of the row-kernel launcher for one (format, mode)
// pair, chosen by the build with -DQMV_INST_FMT=<format struct> and
// -DQMV_INST_MODE=<mode>.  Each pair compiles to its own object, so the
// kernels of the single-token, fused-row, argmax, MoE, gated and
// short-convolution entry points build in parallel.  Without the two macros
// this unit is empty.
#include "qmv_launch_impl.h"

#if defined(QMV_INST_FMT) && defined(QMV_INST_MODE)
namespace qmv {
template hipError_t launch_typed<QMV_INST_FMT, QMV_INST_MODE>(const RowsParams &, hipStream_t,
                                                              int *);
}  // namespace qmv
#endif
