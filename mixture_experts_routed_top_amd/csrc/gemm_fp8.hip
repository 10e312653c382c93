// FP8 E4M3 128-block-scaled grouped GEMMs (not yet enabled: every block_m is
// reported unsupported, so the C ABI rejects the dtype before any launch).
#include "moe_launch.h"

namespace moe {
bool gemm_fp8_supports(int) { return false; }
hipError_t launch_gemm1_fp8(const GemmArgs&, const DeviceInfo&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gemm2_fp8(const GemmArgs&, const DeviceInfo&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace moe
