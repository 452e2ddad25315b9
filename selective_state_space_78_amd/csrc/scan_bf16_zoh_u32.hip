// Scan kernels for bf16 tensors with the zero-order-hold input term, reading u
// in fp32: the convolution prologue's output, which its own pass keeps in fp32.
#define SSM_SCAN_INSTANTIATE
#include "scan_kernels.hpp"

namespace ssm_detail {

hipError_t launch_scan_bf16_zoh_u32(const Plan &pl, const ScanParams &p, int nm, int na, hipStream_t st) {
    return launch_scan_shape<uint16_t, true, true>(pl, p, nm, na, st);
}

}  // namespace ssm_detail
