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
size_t bwd_workspace_bytes(const moe_config&) { return 0; }
hipError_t launch_down_bwd(const moe_config&, const void*, const void*, const void*, const void*, const int32_t*, void*,
                           float*, void*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_swiglu_bwd(const moe_config&, const void*, const void*, const void*, const int32_t*, void*, float*,
                             void*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace moe
