// Launchers of the expert FFN backward GEMMs (kernel in gemm_bwd_kernel.h).
//
//   moe_grouped_down_bwd:   dGU = dSwiGLU(dYp * W2_e^T, stash)   (DGRAD + SwiGLU backward)
//                           dW2_e = dYp_e^T * h_e               (WGRAD, zero for empty experts)
//   moe_grouped_swiglu_bwd: dXp = dGU * W1_e                    (DGRAD)
//                           dW1_e = dGU_e^T * Xp_e              (WGRAD, zero for empty experts)
// bf16 storage only.
#include "gemm_bwd_kernel.h"

namespace moe {

int gemm_persistent_grid(int64_t max_tiles);

size_t bwd_workspace_bytes(const moe_config&) { return 0; }

namespace {

template <int MODE>
hipError_t launch(const gemm::BwdArgs& a, int64_t max_tiles, hipStream_t s) {
    if (max_tiles <= 0) return hipSuccess;
    gemm::grouped_gemm_bwd<MODE><<<gemm_persistent_grid(max_tiles), gemm::kThreads, 0, s>>>(a);
    return hipGetLastError();
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

hipError_t launch_down_bwd(const moe_config& c, const void* dyp, const void* w2, const void* h, const void* stash,
                           const int32_t* offsets, void* dgu, float* dw2, void*, hipStream_t s) {
    if (c.dtype != MOE_BF16) return hipErrorNotSupported;
    const int64_t R = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    gemm::BwdArgs d{(const uint16_t*)dyp, (const uint16_t*)w2, offsets, c.E, (int)R, 0, c.F, c.H,
                    (uint16_t*)dgu, nullptr, (const uint16_t*)stash};
    hipError_t e = launch<gemm::kDgradDswiglu>(d, (R / gemm::kTile + c.E) * cdiv(c.F, gemm::kTile), s);
    if (e != hipSuccess) return e;
    gemm::BwdArgs w{(const uint16_t*)dyp, (const uint16_t*)h, offsets, c.E, (int)R, c.H, c.F, 0,
                    nullptr, dw2, nullptr};
    return launch<gemm::kWgrad>(w, (int64_t)c.E * cdiv(c.H, gemm::kTile) * cdiv(c.F, gemm::kTile), s);
}

hipError_t launch_swiglu_bwd(const moe_config& c, const void* dgu, const void* w1, const void* xp,
                             const int32_t* offsets, void* dxp, float* dw1, void*, hipStream_t s) {
    if (c.dtype != MOE_BF16) return hipErrorNotSupported;
    const int64_t R = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    gemm::BwdArgs d{(const uint16_t*)dgu, (const uint16_t*)w1, offsets, c.E, (int)R, 0, c.H, 2 * c.F,
                    (uint16_t*)dxp, nullptr, nullptr};
    hipError_t e = launch<gemm::kDgrad>(d, (R / gemm::kTile + c.E) * cdiv(c.H, gemm::kTile), s);
    if (e != hipSuccess) return e;
    gemm::BwdArgs w{(const uint16_t*)dgu, (const uint16_t*)xp, offsets, c.E, (int)R, 2 * c.F, c.H, 0,
                    nullptr, dw1, nullptr};
    return launch<gemm::kWgrad>(w, (int64_t)c.E * cdiv(2 * c.F, gemm::kTile) * cdiv(c.H, gemm::kTile), s);
}

}  // namespace moe
