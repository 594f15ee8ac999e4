// Entry points whose kernels are not built yet report "not supported".
#include "moe_internal.h"

namespace moe {

hipError_t launch_swiglu_gemm_mxfp8(const moe_config&, const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*,
                                    const int32_t*, uint8_t*, uint8_t*, uint16_t*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_down_gemm_mxfp8(const moe_config&, const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*,
                                  const int32_t*, uint16_t*, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace moe
