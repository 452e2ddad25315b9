// SSD layer kernels with the zero-order-hold input weight.
#define SSM_SSD_INSTANTIATE
#include "ssd_kernels.hpp"

namespace ssm_detail {

hipError_t launch_ssd_zoh(const SsdParams &p, int P, int N, hipStream_t st) { return launch_ssd_t<true>(p, P, N, st); }

}  // namespace ssm_detail
