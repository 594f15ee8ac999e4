// Top-k weighted combine, and the two gather/scatter steps of the backward.
//
// Combine follows the per-top-k combine of the cudnn-frontend page "Add MoE +
// expert-parallel Python API surface, PyTorch reference, and tests" (Summary)
// and the TransformerEngine page "[JAX] Expert Parallelism: JAX primitives +
// VJPs" (expert outputs summed across the top-k; padded or unused rows are
// never multiplied in, since NaN * 0 would still be NaN).  All three kernels
// are HBM-bound row gathers: one block per token (or per destination row),
// 16-byte vector loads and stores, float32 accumulation, one rounding.
#include "moe_internal.h"

namespace moe {
namespace {

// 8 bfloat16 or 4 float32 per 16-byte vector.
template <bool F32>
struct Vec;
template <>
struct Vec<false> {
    static constexpr int N = 8;
    __device__ static void load(const void* p, int64_t i, float* v) {
        const uint4 q = ((const uint4*)p)[i];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            v[2 * a] = __uint_as_float(w[a] << 16);
            v[2 * a + 1] = __uint_as_float(w[a] & 0xffff0000u);
        }
    }
    __device__ static void store(void* p, int64_t i, const float* v) {
        uint4 q;
        q.x = pack_bf16x2(v[0], v[1]);
        q.y = pack_bf16x2(v[2], v[3]);
        q.z = pack_bf16x2(v[4], v[5]);
        q.w = pack_bf16x2(v[6], v[7]);
        ((uint4*)p)[i] = q;
    }
};
template <>
struct Vec<true> {
    static constexpr int N = 4;
    __device__ static void load(const void* p, int64_t i, float* v) {
        const float4 q = ((const float4*)p)[i];
        v[0] = q.x;
        v[1] = q.y;
        v[2] = q.z;
        v[3] = q.w;
    }
    __device__ static void store(void* p, int64_t i, const float* v) {
        ((float4*)p)[i] = make_float4(v[0], v[1], v[2], v[3]);
    }
};

// y[t] = round(sum_j w[t,j] * Yp[row_map[t,j]]); one block per token.
template <bool F32>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ yp, const int32_t* __restrict__ row_map,
                                                      const float* __restrict__ w, int k, int vec_per_row,
                                                      int64_t n_rows, void* __restrict__ y) {
    using V = Vec<F32>;
    const int64_t t = blockIdx.x;
    for (int c = threadIdx.x; c < vec_per_row; c += blockDim.x) {
        float acc[V::N];
#pragma unroll
        for (int a = 0; a < V::N; ++a) acc[a] = 0.f;
        for (int j = 0; j < k; ++j) {
            const int32_t r = row_map[t * k + j];
            if (r < 0 || r >= n_rows) continue;
            const float wt = w[t * k + j];
            float v[V::N];
            V::load(yp, (int64_t)r * vec_per_row + c, v);
#pragma unroll
            for (int a = 0; a < V::N; ++a) acc[a] = fmaf(wt, v[a], acc[a]);
        }
        V::store(y, t * vec_per_row + c, acc);
    }
}

// dYp[r] = round(w[s] * dy[s / k]) for a real row, 0 for a padding row.
template <bool F32>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const void* __restrict__ dy,
                                                          const int32_t* __restrict__ src_map,
                                                          const int32_t* __restrict__ offsets, int E,
                                                          const float* __restrict__ w, int k, int vec_per_row,
                                                          int64_t n_routes, void* __restrict__ dyp) {
    using V = Vec<F32>;
    const int64_t r = blockIdx.x;
    if (r >= offsets[E]) return;
    int32_t s = src_map[r];  // -1 or a route index t*k+j (< T*k)
    if (s >= n_routes) s = -1;
    const float wt = s >= 0 ? w[s] : 0.f;
    for (int c = threadIdx.x; c < vec_per_row; c += blockDim.x) {
        float v[V::N];
        if (s >= 0) {
            V::load(dy, (int64_t)(s / k) * vec_per_row + c, v);
#pragma unroll
            for (int a = 0; a < V::N; ++a) v[a] *= wt;
        } else {
#pragma unroll
            for (int a = 0; a < V::N; ++a) v[a] = 0.f;
        }
        V::store(dyp, r * vec_per_row + c, v);
    }
}

// dx[t] = round(sum_j dXp[row_map[t,j]]).
template <bool F32>
__global__ __launch_bounds__(256) void permute_bwd_kernel(const void* __restrict__ dxp,
                                                          const int32_t* __restrict__ row_map, int k,
                                                          int vec_per_row, int64_t n_rows, void* __restrict__ dx) {
    using V = Vec<F32>;
    const int64_t t = blockIdx.x;
    for (int c = threadIdx.x; c < vec_per_row; c += blockDim.x) {
        float acc[V::N];
#pragma unroll
        for (int a = 0; a < V::N; ++a) acc[a] = 0.f;
        for (int j = 0; j < k; ++j) {
            const int32_t r = row_map[t * k + j];
            if (r < 0 || r >= n_rows) continue;
            float v[V::N];
            V::load(dxp, (int64_t)r * vec_per_row + c, v);
#pragma unroll
            for (int a = 0; a < V::N; ++a) acc[a] += v[a];
        }
        V::store(dx, t * vec_per_row + c, acc);
    }
}

int block_for(int vec_per_row) {
    int b = 64;
    while (b < vec_per_row && b < 256) b *= 2;
    return b;
}

}  // namespace

hipError_t launch_combine(const moe_config& c, const void* yp, const int32_t* row_map, const float* w, void* y,
                          hipStream_t s) {
    if (c.T == 0) return hipSuccess;
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    const bool f32 = c.dtype == MOE_F32;
    const int vpr = c.H / (f32 ? 4 : 8);
    if (f32)
        combine_kernel<true><<<c.T, block_for(vpr), 0, s>>>(yp, row_map, w, c.k, vpr, R_cap, y);
    else
        combine_kernel<false><<<c.T, block_for(vpr), 0, s>>>(yp, row_map, w, c.k, vpr, R_cap, y);
    return hipGetLastError();
}

hipError_t launch_combine_bwd(const moe_config& c, const void* dy, const int32_t* src_map, const int32_t* offsets,
                              const float* w, void* dyp, hipStream_t s) {
    const int64_t rows = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    if (rows == 0) return hipSuccess;
    const bool f32 = c.dtype == MOE_F32;
    const int vpr = c.H / (f32 ? 4 : 8);
    if (f32)
        combine_bwd_kernel<true><<<rows, block_for(vpr), 0, s>>>(dy, src_map, offsets, c.E, w, c.k, vpr, (int64_t)c.T * c.k, dyp);
    else
        combine_bwd_kernel<false><<<rows, block_for(vpr), 0, s>>>(dy, src_map, offsets, c.E, w, c.k, vpr, (int64_t)c.T * c.k, dyp);
    return hipGetLastError();
}

hipError_t launch_permute_bwd(const moe_config& c, const void* dxp, const int32_t* row_map, void* dx,
                              hipStream_t s) {
    if (c.T == 0) return hipSuccess;
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    const bool f32 = c.dtype == MOE_F32;
    const int vpr = c.H / (f32 ? 4 : 8);
    if (f32)
        permute_bwd_kernel<true><<<c.T, block_for(vpr), 0, s>>>(dxp, row_map, c.k, vpr, R_cap, dx);
    else
        permute_bwd_kernel<false><<<c.T, block_for(vpr), 0, s>>>(dxp, row_map, c.k, vpr, R_cap, dx);
    return hipGetLastError();
}

}  // namespace moe
