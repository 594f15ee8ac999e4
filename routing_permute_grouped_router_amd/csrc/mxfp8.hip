// MXFP8 (OCP E4M3 elements, E8M0 scale per 32 consecutive elements) and
// MXFP4 (OCP E2M1 elements, packed two per byte, the same scales).
//
// The block-32 scaled format is the MXFP8 BlockScaledTensor of the
// cudnn-frontend page "Add MoE + expert-parallel Python API surface, PyTorch
// reference, and tests" (review comment on BlockScaledTensor) and the grouped
// MXFP8 quantisation listed by the tracking issue "MoE training
// optimization".  The conversion rule is the public OCP Microscaling (MX)
// Formats v1.0 one: shared exponent floor(log2(amax)) - 8 (E4M3's largest
// exponent), clamped to the E8M0 range; elements rounded to nearest even,
// saturating at +-448.  MXFP4 follows the same rule with E2M1 elements
// (shared exponent floor(log2(amax)) - 2, saturating at +-6): the MX analogue
// of the NVFP4 recipe named by the same two pages, on CDNA4's scaled matrix
// cores.
#include "moe_internal.h"
#include "mxfp8.h"

namespace moe {
namespace {

// 8 lanes per block of 32 values, 4 values (16 bytes) per lane.
__global__ __launch_bounds__(256) void quantize_mxfp8_kernel(const float* __restrict__ in, int64_t n_blocks,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t blk = gid >> 3;
    const bool live = blk < n_blocks;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) v = ((const float4*)in)[gid];
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if (!live) return;
    const int se = mx_shared_exp(amax);
    const uint32_t packed = (uint32_t)e4m3_rne(ldexpf(v.x, -se)) | ((uint32_t)e4m3_rne(ldexpf(v.y, -se)) << 8) |
                            ((uint32_t)e4m3_rne(ldexpf(v.z, -se)) << 16) |
                            ((uint32_t)e4m3_rne(ldexpf(v.w, -se)) << 24);
    ((uint32_t*)codes)[gid] = packed;
    if ((gid & 7) == 0) scales[blk] = (uint8_t)(se + 127);
}

// 4 lanes per block of 32 values, 8 values (two float4 in, four packed code
// bytes out) per lane.
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const float* __restrict__ in, int64_t n_blocks,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t blk = gid >> 2;
    const bool live = blk < n_blocks;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (live) {
        a = ((const float4*)in)[2 * gid];
        b = ((const float4*)in)[2 * gid + 1];
    }
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    if (!live) return;
    const int se = mx4_shared_exp(amax);
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) packed |= (uint32_t)e2m1_rne(ldexpf(v[j], -se)) << (4 * j);
    ((uint32_t*)codes)[gid] = packed;
    if ((gid & 3) == 0) scales[blk] = (uint8_t)(se + 127);
}

}  // namespace

hipError_t launch_quantize_mxfp4(const float* in, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s) {
    const int64_t n_blocks = rows * (cols / kMxBlock);
    if (n_blocks == 0) return hipSuccess;
    const int64_t threads = n_blocks * 4;
    quantize_mxfp4_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(in, n_blocks, codes, scales);
    return hipGetLastError();
}

hipError_t launch_quantize_mxfp8(const float* in, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s) {
    const int64_t n_blocks = rows * (cols / kMxBlock);
    if (n_blocks == 0) return hipSuccess;
    const int64_t threads = n_blocks * 8;
    quantize_mxfp8_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(in, n_blocks, codes, scales);
    return hipGetLastError();
}

}  // namespace moe

// ---------------------------------------------------------------- GEMMs
#include "gemm_mxfp8_kernel.h"

namespace moe {

int gemm_persistent_grid(int64_t max_tiles);

namespace {

// Zeroes the 8 work-queue counters (a kernel rather than a memset node, so
// the calls stay safe to capture in a graph).
__global__ void zero_mx_sched_kernel(int* sched) {
    if (threadIdx.x < gemm::kXcds) sched[threadIdx.x] = 0;
}

int64_t rows_cap(const moe_config& c) { return (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1); }

}  // namespace

// The instance of a GEMM kernel for the epilogue variant the arguments ask
// for: row weights (bit 1), SwiGLU clamp (bit 2).
template <bool SWIGLU, int G, bool F4>
void mx_launch(const gemm::MxArgs& a, int64_t max_tiles, hipStream_t s) {
    const int ep = (a.row_w ? 1 : 0) | (SWIGLU && a.lim < INFINITY ? 2 : 0);
    const unsigned grid = gemm_persistent_grid(max_tiles);
    if (ep == 0) gemm::grouped_gemm_mxfp8<SWIGLU, G, 0, F4><<<grid, gemm::kThreads, 0, s>>>(a);
    else if (ep == 1) gemm::grouped_gemm_mxfp8<SWIGLU, G, 1, F4><<<grid, gemm::kThreads, 0, s>>>(a);
    else if constexpr (SWIGLU) {
        if (ep == 2) gemm::grouped_gemm_mxfp8<SWIGLU, G, 2, F4><<<grid, gemm::kThreads, 0, s>>>(a);
        else gemm::grouped_gemm_mxfp8<SWIGLU, G, 3, F4><<<grid, gemm::kThreads, 0, s>>>(a);
    }
}

// The instance for the format and K: E2M1 loads the scales of two stages
// (512 values) per 16-byte row load, K a multiple of 512 (host-checked); E4M3
// those of four stages when K is a multiple of 512, else one word per stage.
template <bool SWIGLU>
void mx_dispatch(const moe_config& c, const gemm::MxArgs& a, int64_t max_tiles, hipStream_t s) {
    if (c.dtype == MOE_MXFP4) mx_launch<SWIGLU, 2, true>(a, max_tiles, s);
    else if (a.K % 512 == 0) mx_launch<SWIGLU, 4, false>(a, max_tiles, s);
    else mx_launch<SWIGLU, 1, false>(a, max_tiles, s);
}

size_t gemm_mxfp8_ws_bytes(const moe_config& c) { return c.dtype == MOE_MXFP8 || c.dtype == MOE_MXFP4 ? 256 : 0; }

hipError_t launch_swiglu_gemm_mxfp8(const moe_config& c, const uint8_t* xp, const uint8_t* xp_scale,
                                    const uint8_t* w1, const uint8_t* w1_scale, const int32_t* offsets, uint8_t* h,
                                    uint8_t* h_scale, uint16_t* stash, const int32_t* src_map,
                                    const int32_t* counts, const float* row_w, void* ws, hipStream_t s) {
    const int64_t max_tiles = (rows_cap(c) / gemm::kTile + c.E) * ((c.F + 127) / 128);
    if (max_tiles == 0) return hipSuccess;
    gemm::MxArgs a{xp, xp_scale, w1, w1_scale, offsets, c.E, c.H, (int)rows_cap(c), c.F, 2 * c.F, h, h_scale,
                   nullptr, stash, (int*)ws, src_map, counts, c.k, row_w,
                   c.swiglu_limit > 0.f ? c.swiglu_limit : INFINITY};
    zero_mx_sched_kernel<<<1, 64, 0, s>>>(a.sched);
    mx_dispatch<true>(c, a, max_tiles, s);
    return hipGetLastError();
}

hipError_t launch_down_gemm_mxfp8(const moe_config& c, const uint8_t* h, const uint8_t* h_scale, const uint8_t* w2,
                                  const uint8_t* w2_scale, const int32_t* offsets, uint16_t* yp, const float* row_w,
                                  void* ws, hipStream_t s) {
    const int64_t max_tiles = (rows_cap(c) / gemm::kTile + c.E) * ((c.H + gemm::kTile - 1) / gemm::kTile);
    if (max_tiles == 0) return hipSuccess;
    gemm::MxArgs a{h, h_scale, w2, w2_scale, offsets, c.E, c.F, (int)rows_cap(c), c.H, c.H, nullptr, nullptr,
                   yp, nullptr, (int*)ws, nullptr, nullptr, 1, row_w, INFINITY};
    zero_mx_sched_kernel<<<1, 64, 0, s>>>(a.sched);
    mx_dispatch<false>(c, a, max_tiles, s);
    return hipGetLastError();
}

}  // namespace moe
