// Backward kernels for bf16 inputs, zero-order-hold input term.
#define SSM_SCAN_INSTANTIATE
#define SSM_BWD_INSTANTIATE
#include "bwd_kernels.hpp"

namespace ssm_detail {
hipError_t launch_bwd_bf16_zoh(const BwdShape &sh, const BwdParams &p, hipStream_t st) {
    return launch_bwd_shape<uint16_t, true>(sh, p, st);
}
}  // namespace ssm_detail
