// MXFP4-weight x MXFP8-activation grouped GEMMs (not yet enabled: every
// block_m is reported unsupported, so the C ABI rejects the dtype).
#include "moe_launch.h"

namespace moe {
bool gemm_mx_supports(int) { return false; }
hipError_t launch_gemm1_mx(const GemmArgs&, const DeviceInfo&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gemm2_mx(const GemmArgs&, const DeviceInfo&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace moe
