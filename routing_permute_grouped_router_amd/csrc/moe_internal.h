// Internal declarations of the MoE HIP library (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;              // CDNA wavefront width
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 64;
constexpr int kMxBlock = 32;

// ----------------------------------------------------------------- numerics
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round-to-nearest-even float32 -> bfloat16 (NaN stays a quiet NaN), with the
// CDNA4 conversion instruction v_cvt_pk_bf16_f32.  It gives the same bits as
// the integer rule ((u + 0x7fff + ((u >> 16) & 1)) >> 16, NaN -> (u >> 16) |
// 0x40), which was checked on 2^24 bit patterns including ties, subnormals,
// infinities and NaNs.
typedef __bf16 moe_bf16x2 __attribute__((ext_vector_type(2)));
typedef float moe_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((moe_f32x2){lo, hi}, moe_bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu); }

// silu(g) = g * sigmoid(g), with the hardware exponential and reciprocal (a
// few float32 ulps; the result is rounded to bf16 or quantised afterwards).
__device__ __forceinline__ float sigmoid_fast(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ __forceinline__ float silu(float g) { return g * sigmoid_fast(g); }

// --------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// --------------------------------------------------------- errors
// Sets the calling thread's moe_last_error() message and returns s.
moe_status set_error(moe_status s, const char* fmt, ...);

// --------------------------------------------------------- host launchers
// Each returns hipSuccess or the launch error; arguments were validated by
// the API layer.
hipError_t launch_route(const moe_config& c, const float* logits, const float* bias, int32_t* idx, float* w,
                        hipStream_t s);

// Grouping and permutation (xp null: the grouping only).  ws holds
// group_n_chunks(T, E) * E int32 (per-chunk expert counts).
int group_n_chunks(int T, int E);
hipError_t launch_group(const moe_config& c, const int32_t* idx, const void* x, const uint8_t* x_scale, void* xp,
                        uint8_t* xp_scale, int32_t* counts, int32_t* offsets, int32_t* row_map, int32_t* src_map,
                        int32_t* err, int32_t* ws, hipStream_t s);

hipError_t launch_combine(const moe_config& c, const void* yp, const int32_t* row_map, const float* w, void* y,
                          hipStream_t s);
hipError_t launch_combine_bwd(const moe_config& c, const void* dy, const int32_t* row_map, const int32_t* src_map,
                              const int32_t* offsets, const float* w, void* dyp, hipStream_t s);
hipError_t launch_permute_bwd(const moe_config& c, const void* dxp, const int32_t* row_map, void* dx,
                              hipStream_t s);
// Per-row routing weights for the epilogue placements: row_w[r] =
// w[src_map[r]] for r < R_cap, 0 for unfilled rows and for the kRowWeightPad
// rows after R_cap (a 256-row tile reads its rows' weights without a bound).
constexpr int kRowWeightPad = 256;
hipError_t launch_row_weights(const moe_config& c, const int32_t* src_map, const float* w, float* row_w,
                              hipStream_t s);
hipError_t launch_route_bwd(const moe_config& c, const void* dy, const void* yp, const float* logits,
                            const int32_t* idx, const int32_t* row_map, float* dw, float* dlogits, hipStream_t s);

// Grouped GEMMs.
// ws: gemm_bf16_ws_bytes(c) bytes (work-queue counters and the partial sums
// of K-split tiles).
size_t gemm_bf16_ws_bytes(const moe_config& c);
// Gate/up GEMMs: with src_map and counts non-null, xp is x [T,H] (+ x_scale)
// and row r of the grouped operand is x[src_map[r] / k] (the gather form).
// row_w (optional, from launch_row_weights): each output row r is scaled by
// row_w[r] before it is stored (h for the gate/up GEMMs, Yp for the down).
hipError_t launch_swiglu_gemm_bf16(const moe_config& c, const uint16_t* xp, const uint16_t* w1,
                                   const int32_t* offsets, uint16_t* h, uint16_t* stash, const int32_t* src_map,
                                   const int32_t* counts, const float* row_w, void* ws, hipStream_t s);
hipError_t launch_down_gemm_bf16(const moe_config& c, const uint16_t* h, const uint16_t* w2, const int32_t* offsets,
                                 uint16_t* yp, const float* row_w, void* ws, hipStream_t s);
hipError_t launch_swiglu_gemm_f32(const moe_config& c, const float* xp, const float* w1, const int32_t* offsets,
                                  float* h, float* stash, const int32_t* src_map, const int32_t* counts,
                                  const float* row_w, hipStream_t s);
hipError_t launch_down_gemm_f32(const moe_config& c, const float* h, const float* w2, const int32_t* offsets,
                                float* yp, const float* row_w, hipStream_t s);

// MXFP8
hipError_t launch_quantize_mxfp4(const float* in, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s);
hipError_t launch_quantize_mxfp8(const float* in, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s);
// Workspace of the MXFP8 GEMMs: their 8 work-queue counters.
size_t gemm_mxfp8_ws_bytes(const moe_config& c);
hipError_t launch_swiglu_gemm_mxfp8(const moe_config& c, const uint8_t* xp, const uint8_t* xp_scale,
                                    const uint8_t* w1, const uint8_t* w1_scale, const int32_t* offsets, uint8_t* h,
                                    uint8_t* h_scale, uint16_t* stash, const int32_t* src_map,
                                    const int32_t* counts, const float* row_w, void* ws, hipStream_t s);
hipError_t launch_down_gemm_mxfp8(const moe_config& c, const uint8_t* h, const uint8_t* h_scale, const uint8_t* w2,
                                  const uint8_t* w2_scale, const int32_t* offsets, uint16_t* yp, const float* row_w,
                                  void* ws, hipStream_t s);

// Backward GEMMs (bf16 / f32 storage).
size_t bwd_workspace_bytes(const moe_config& c);
hipError_t launch_down_bwd(const moe_config& c, const void* dyp, const void* w2, const void* h, const void* stash,
                           const int32_t* offsets, void* dgu, float* dw2, void* ws, hipStream_t s);
hipError_t launch_swiglu_bwd(const moe_config& c, const void* dgu, const void* w1, const void* xp,
                             const int32_t* offsets, void* dxp, float* dw1, void* ws, hipStream_t s);

}  // namespace moe
