// Quantised weight formats (fp8 128x128 block scales, MXFP4 x fp8).
#include "common.h"
#include "launch.h"

namespace moe {
moe_status launch_quant_x(const FfnArgs&, hipStream_t) { return MOE_E_UNSUPPORTED; }
moe_status launch_gemm_fp8(const FfnArgs&, int, hipStream_t) { return MOE_E_UNSUPPORTED; }
moe_status launch_gemm_mxfp4(const FfnArgs&, int, hipStream_t) { return MOE_E_UNSUPPORTED; }
}  // namespace moe
