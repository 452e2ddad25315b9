// SSD layer kernels with the simplified (dt) input weight.
#define SSM_SSD_INSTANTIATE
#include "ssd_kernels.hpp"

namespace ssm_detail {

hipError_t launch_ssd_euler(const SsdParams &p, int P, int N, hipStream_t st) { return launch_ssd_t<false>(p, P, N, st); }

}  // namespace ssm_detail
