// Grouped FP8 (E4M3FN, 1x128 / 128x128 block-scaled) expert GEMMs.
#include "moe_internal.h"

namespace moe {

hipError_t launch_gemm_fp8_swiglu(const GemmOperands&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gemm_fp8_down(const GemmOperands&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace moe
