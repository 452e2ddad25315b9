// Backward kernels for f32 inputs, simplified (delta B u) input term.
#define SSM_SCAN_INSTANTIATE
#define SSM_BWD_INSTANTIATE
#include "bwd_kernels.hpp"

namespace ssm_detail {
hipError_t launch_bwd_f32_euler(const BwdShape &sh, const BwdParams &p, hipStream_t st) {
    return launch_bwd_shape<float, false>(sh, p, st);
}
}  // namespace ssm_detail
