// Grouped bf16 GEMMs of the expert FFN forward on CDNA4 matrix cores.
//
// The gate/up projection fused with SwiGLU and the down projection, per the
// Diagram of the TransformerEngine page "[Draft][JAX] MoE block optimization"
// (fused grouped GEMM and SwiGLU, then the down projection) and the
// cudnn-frontend page "Add MoE + expert-parallel Python API surface, PyTorch
// reference, and tests" (silu(gate) * up).  Group sizes come from the device
// `offsets` buffer, as the TransformerEngine page "[JAX] Expert Parallelism:
// JAX primitives + VJPs" does with its device token counts (commit "plumb
// token_counts to grouped_gemm ..."); empty experts own no tiles and ragged
// tails are masked.  The kernel itself is in gemm_bf16_kernel.h.
#include <algorithm>

#include "gemm_bf16_kernel.h"

namespace moe {
namespace {

// Tuned on MI355X with the Mixtral-shaped and fine-grained layers.
constexpr int kSwizzle = 0, kGroupM = 4;

int g_num_cus = 0;

int num_cus() {
    if (g_num_cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            g_num_cus = n;
        else
            g_num_cus = 256;
    }
    return g_num_cus;
}

}  // namespace

int gemm_persistent_grid(int64_t max_tiles) {
    int g = num_cus();
    g = (g / gemm::kXcds) * gemm::kXcds;
    if (g < gemm::kXcds) g = gemm::kXcds;
    const int64_t need = ((max_tiles + gemm::kXcds - 1) / gemm::kXcds) * gemm::kXcds;
    return (int)std::min<int64_t>(g, std::max<int64_t>(need, gemm::kXcds));
}

hipError_t launch_swiglu_gemm_bf16(const moe_config& c, const uint16_t* xp, const uint16_t* w1,
                                   const int32_t* offsets, uint16_t* h, uint16_t* stash, hipStream_t s) {
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    const int64_t max_tiles = (R_cap / gemm::kTile + c.E) * ((c.F + 127) / 128);
    if (max_tiles == 0) return hipSuccess;
    gemm::Args a{xp, w1, offsets, c.E, c.H, (int)R_cap, c.F, 2 * c.F, h, stash};
    gemm::grouped_gemm_bf16<true, kSwizzle, kGroupM>
        <<<gemm_persistent_grid(max_tiles), gemm::kThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_down_gemm_bf16(const moe_config& c, const uint16_t* h, const uint16_t* w2, const int32_t* offsets,
                                 uint16_t* yp, hipStream_t s) {
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    const int64_t max_tiles = (R_cap / gemm::kTile + c.E) * ((c.H + gemm::kTile - 1) / gemm::kTile);
    if (max_tiles == 0) return hipSuccess;
    gemm::Args a{h, w2, offsets, c.E, c.F, (int)R_cap, c.H, c.H, yp, nullptr};
    gemm::grouped_gemm_bf16<false, kSwizzle, kGroupM>
        <<<gemm_persistent_grid(max_tiles), gemm::kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
