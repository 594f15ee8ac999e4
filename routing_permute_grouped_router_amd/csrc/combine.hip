// Top-k weighted combine, and the two gather/scatter steps of the backward.
//
// Combine follows the per-top-k combine of the cudnn-frontend page "Add MoE +
// expert-parallel Python API surface, PyTorch reference, and tests" (Summary)
// and the TransformerEngine page "[JAX] Expert Parallelism: JAX primitives +
// VJPs" (expert outputs summed across the top-k; padded or unused rows are
// never multiplied in, since NaN * 0 would still be NaN).  All kernels here
// are HBM-bound row moves with 16-byte vector loads and stores: the combine
// and the permute backward gather a token's k rows (one block per token,
// float32 accumulation, one rounding); the combine backward reads each token's
// gradient row once and scatters it to the token's k rows.
#include "moe_internal.h"

namespace moe {
namespace {

// 8 bfloat16 or 4 float32 per 16-byte vector.
template <bool F32>
struct Vec;
template <>
struct Vec<false> {
    static constexpr int N = 8;
    template <bool NT = false>
    __device__ static void load(const void* p, int64_t i, float* v) {
        uint4 q;
        if (NT) {
            const uint32_t* a = (const uint32_t*)((const uint4*)p + i);
            q = make_uint4(__builtin_nontemporal_load(a), __builtin_nontemporal_load(a + 1),
                           __builtin_nontemporal_load(a + 2), __builtin_nontemporal_load(a + 3));
        } else {
            q = ((const uint4*)p)[i];
        }
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            v[2 * a] = __uint_as_float(w[a] << 16);
            v[2 * a + 1] = __uint_as_float(w[a] & 0xffff0000u);
        }
    }
    template <bool NT = false>
    __device__ static void store(void* p, int64_t i, const float* v) {
        uint4 q;
        q.x = pack_bf16x2(v[0], v[1]);
        q.y = pack_bf16x2(v[2], v[3]);
        q.z = pack_bf16x2(v[4], v[5]);
        q.w = pack_bf16x2(v[6], v[7]);
        if (NT) {
            uint32_t* a = (uint32_t*)((uint4*)p + i);
            __builtin_nontemporal_store(q.x, a);
            __builtin_nontemporal_store(q.y, a + 1);
            __builtin_nontemporal_store(q.z, a + 2);
            __builtin_nontemporal_store(q.w, a + 3);
        } else {
            ((uint4*)p)[i] = q;
        }
    }
};
template <>
struct Vec<true> {
    static constexpr int N = 4;
    template <bool NT = false>
    __device__ static void load(const void* p, int64_t i, float* v) {
        const float4 q = ((const float4*)p)[i];
        v[0] = q.x;
        v[1] = q.y;
        v[2] = q.z;
        v[3] = q.w;
    }
    template <bool NT = false>
    __device__ static void store(void* p, int64_t i, const float* v) {
        ((float4*)p)[i] = make_float4(v[0], v[1], v[2], v[3]);
    }
};

// Gathers read the routes of a token in groups of G (the smallest of 1, 2, 4,
// 8 that covers k, 8 for larger k): the group's row indices first, then all
// of its row loads, unconditionally (a route without a valid row reads row 0
// and is masked out), then the accumulation in ascending j.  Each lane then has
// G 16-byte loads in flight instead of one.
template <int G>
__device__ __forceinline__ void gather_rows(const int32_t* __restrict__ row_map, int64_t t, int k, int j0,
                                            int64_t n_rows, int32_t (&r)[G], bool (&ok)[G]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int j = j0 + g;
        r[g] = j < k ? row_map[t * k + j] : -1;
        ok[g] = r[g] >= 0 && r[g] < n_rows;
        if (!ok[g]) r[g] = 0;
    }
}

// y[t] = round(sum_j w[t,j] * Yp[row_map[t,j]]); one block per token.  w null:
// the weights were applied in an expert epilogue, the routes are summed.
template <bool F32, int G, bool TWO>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ yp, const int32_t* __restrict__ row_map,
                                                      const float* __restrict__ w, int k, int vec_per_row,
                                                      int64_t n_rows, void* __restrict__ y) {
    using V = Vec<F32>;
    const int64_t t = blockIdx.x;
    // TWO (rows longer than the block): two vectors of the row per thread at
    // a time (columns c and c + blockDim), so 2 G row loads are in flight per
    // lane; otherwise one (fewer registers, more blocks resident)
    for (int c0 = threadIdx.x; c0 < vec_per_row; c0 += (TWO ? 2 : 1) * blockDim.x) {
        const int c1 = c0 + blockDim.x;
        const bool two = TWO && c1 < vec_per_row;
        float acc0[V::N], acc1[V::N];
#pragma unroll
        for (int a = 0; a < V::N; ++a) acc0[a] = acc1[a] = 0.f;
        for (int j0 = 0; j0 < k; j0 += G) {
            int32_t r[G];
            bool ok[G];
            float v0[G][V::N], v1[G][V::N];
            gather_rows<G>(row_map, t, k, j0, n_rows, r, ok);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                V::template load<true>(yp, (int64_t)r[g] * vec_per_row + c0, v0[g]);
                if (two) V::template load<true>(yp, (int64_t)r[g] * vec_per_row + c1, v1[g]);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float wt = ok[g] ? (w ? w[t * k + j0 + g] : 1.f) : 0.f;
#pragma unroll
                for (int a = 0; a < V::N; ++a) {
                    acc0[a] = ok[g] ? fmaf(wt, v0[g][a], acc0[a]) : acc0[a];
                    acc1[a] = ok[g] ? fmaf(wt, v1[g][a], acc1[a]) : acc1[a];
                }
            }
        }
        // y is not read again here: non-temporal stores keep it from
        // displacing cached lines
        V::template store<true>(y, t * vec_per_row + c0, acc0);
        if (two) V::template store<true>(y, t * vec_per_row + c1, acc1);
    }
}

// dYp[row_map[t,j]] = round(w[t,j] * dy[t]): each token's gradient row is read
// once and written to its k rows; tpb tokens per block when a row is shorter
// than the block.
template <bool F32>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const void* __restrict__ dy,
                                                          const int32_t* __restrict__ row_map,
                                                          const float* __restrict__ w, int T, int k,
                                                          int vec_per_row, int tpb, int64_t n_rows,
                                                          void* __restrict__ dyp) {
    using V = Vec<F32>;
    const int t0 = blockIdx.x * tpb;
    const int n = min(tpb, T - t0) * vec_per_row;
    for (int q = threadIdx.x; q < n; q += blockDim.x) {
        const int t = t0 + q / vec_per_row;
        const int c = q % vec_per_row;
        float v[V::N], o[V::N];
        V::load(dy, (int64_t)t * vec_per_row + c, v);
        for (int j = 0; j < k; ++j) {
            const int32_t r = row_map[(int64_t)t * k + j];
            if (r < 0 || r >= n_rows) continue;
            const float wt = w[(int64_t)t * k + j];
#pragma unroll
            for (int a = 0; a < V::N; ++a) o[a] = v[a] * wt;
            V::template store<true>(dyp, (int64_t)r * vec_per_row + c, o);
        }
    }
}

// Rows r < offsets[E] that carry no route (src_map[r] outside [0, n_routes):
// the padding of a group) get dYp[r] = 0.  A block checks 256 rows, one per
// thread, and then clears its padding rows (usually none) together.
template <bool F32>
__global__ __launch_bounds__(256) void zero_unrouted_rows_kernel(const int32_t* __restrict__ src_map,
                                                                 const int32_t* __restrict__ offsets, int E,
                                                                 int64_t n_routes, int vec_per_row, int64_t n_rows,
                                                                 void* __restrict__ dyp) {
    using V = Vec<F32>;
    __shared__ int32_t pad[256];
    __shared__ int n_pad;
    if (threadIdx.x == 0) n_pad = 0;
    __syncthreads();
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (r < min((int64_t)offsets[E], n_rows)) {
        const int32_t s = src_map[r];
        if (s < 0 || s >= n_routes) pad[atomicAdd(&n_pad, 1)] = (int32_t)(r - (int64_t)blockIdx.x * 256);
    }
    __syncthreads();
    float z[V::N];
#pragma unroll
    for (int a = 0; a < V::N; ++a) z[a] = 0.f;
    const int n = n_pad * vec_per_row;
    for (int q = threadIdx.x; q < n; q += 256)
        V::store(dyp, ((int64_t)blockIdx.x * 256 + pad[q / vec_per_row]) * vec_per_row + q % vec_per_row, z);
}

// dx[t] = round(sum_j dXp[row_map[t,j]]).
template <bool F32, int G>
__global__ __launch_bounds__(256) void permute_bwd_kernel(const void* __restrict__ dxp,
                                                          const int32_t* __restrict__ row_map, int k,
                                                          int vec_per_row, int64_t n_rows, void* __restrict__ dx) {
    using V = Vec<F32>;
    const int64_t t = blockIdx.x;
    for (int c = threadIdx.x; c < vec_per_row; c += blockDim.x) {
        float acc[V::N];
#pragma unroll
        for (int a = 0; a < V::N; ++a) acc[a] = 0.f;
        for (int j0 = 0; j0 < k; j0 += G) {
            int32_t r[G];
            bool ok[G];
            float v[G][V::N];
            gather_rows<G>(row_map, t, k, j0, n_rows, r, ok);
#pragma unroll
            for (int g = 0; g < G; ++g) V::template load<true>(dxp, (int64_t)r[g] * vec_per_row + c, v[g]);
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int a = 0; a < V::N; ++a) acc[a] = ok[g] ? acc[a] + v[g][a] : acc[a];
        }
        V::store(dx, t * vec_per_row + c, acc);
    }
}

// Launch a gather kernel template K<F32, G> with G chosen from k.
#define MOE_GATHER_LAUNCH(KERNEL, F32, k, grid, block, s, ...)                                            \
    do {                                                                                                 \
        if ((k) <= 1) KERNEL<F32, 1><<<grid, block, 0, s>>>(__VA_ARGS__);                                \
        else if ((k) <= 2) KERNEL<F32, 2><<<grid, block, 0, s>>>(__VA_ARGS__);                           \
        else if ((k) <= 4) KERNEL<F32, 4><<<grid, block, 0, s>>>(__VA_ARGS__);                           \
        else KERNEL<F32, 8><<<grid, block, 0, s>>>(__VA_ARGS__);                                         \
    } while (0)

template <bool F32, bool TWO>
hipError_t combine_t(int k, int T, int b, hipStream_t s, const void* yp, const int32_t* row_map, const float* w,
                     int vpr, int64_t R_cap, void* y) {
    if (k <= 1) combine_kernel<F32, 1, TWO><<<T, b, 0, s>>>(yp, row_map, w, k, vpr, R_cap, y);
    else if (k <= 2) combine_kernel<F32, 2, TWO><<<T, b, 0, s>>>(yp, row_map, w, k, vpr, R_cap, y);
    else if (k <= 4) combine_kernel<F32, 4, TWO><<<T, b, 0, s>>>(yp, row_map, w, k, vpr, R_cap, y);
    else combine_kernel<F32, 8, TWO><<<T, b, 0, s>>>(yp, row_map, w, k, vpr, R_cap, y);
    return hipGetLastError();
}

int block_for(int vec_per_row) {
    int b = 64;
    while (b < vec_per_row && b < 256) b *= 2;
    return b;
}

}  // namespace

namespace {
// row_w[r] = w[src_map[r]] (the routing weight of the route in row r), 0 for
// rows no route fills; rows [R_cap, n_alloc) are set to 0 as well.
__global__ __launch_bounds__(256) void row_weights_kernel(const int32_t* __restrict__ src_map,
                                                          const float* __restrict__ w, int64_t n_rows,
                                                          int64_t n_alloc, int64_t n_routes, float* __restrict__ row_w) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= n_alloc) return;
    const int32_t s = r < n_rows ? src_map[r] : -1;
    row_w[r] = (s >= 0 && s < n_routes) ? w[s] : 0.f;
}
}  // namespace

hipError_t launch_row_weights(const moe_config& c, const int32_t* src_map, const float* w, float* row_w,
                              hipStream_t s) {
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    const int64_t n = R_cap + kRowWeightPad;
    row_weights_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(src_map, w, R_cap, n, (int64_t)c.T * c.k, row_w);
    return hipGetLastError();
}

hipError_t launch_combine(const moe_config& c, const void* yp, const int32_t* row_map, const float* w, void* y,
                          hipStream_t s) {
    if (c.T == 0) return hipSuccess;
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    const bool f32 = c.dtype == MOE_F32;
    const int vpr = c.H / (f32 ? 4 : 8);
    const int b = block_for(vpr);
    // two vectors per thread pay off for short top-k only (with k = 8 the
    // doubled registers cost more resident blocks than the loads gain)
    const bool two = vpr > b && c.k <= 4;
    if (f32) {
        if (two) return combine_t<true, true>(c.k, c.T, b, s, yp, row_map, w, vpr, R_cap, y);
        return combine_t<true, false>(c.k, c.T, b, s, yp, row_map, w, vpr, R_cap, y);
    }
    if (two) return combine_t<false, true>(c.k, c.T, b, s, yp, row_map, w, vpr, R_cap, y);
    return combine_t<false, false>(c.k, c.T, b, s, yp, row_map, w, vpr, R_cap, y);
}

hipError_t launch_combine_bwd(const moe_config& c, const void* dy, const int32_t* row_map, const int32_t* src_map,
                              const int32_t* offsets, const float* w, void* dyp, hipStream_t s) {
    const int64_t rows = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    if (rows == 0) return hipSuccess;
    const bool f32 = c.dtype == MOE_F32;
    const int vpr = c.H / (f32 ? 4 : 8);
    const int tpb = vpr >= 256 ? 1 : (256 + vpr - 1) / vpr;
    const int64_t n_routes = (int64_t)c.T * c.k;
    const unsigned zgrid = (unsigned)((rows + 255) / 256);
    if (f32) {
        zero_unrouted_rows_kernel<true><<<zgrid, 256, 0, s>>>(src_map, offsets, c.E, n_routes, vpr, rows, dyp);
        if (c.T > 0)
            combine_bwd_kernel<true><<<(c.T + tpb - 1) / tpb, 256, 0, s>>>(dy, row_map, w, c.T, c.k, vpr, tpb, rows, dyp);
    } else {
        zero_unrouted_rows_kernel<false><<<zgrid, 256, 0, s>>>(src_map, offsets, c.E, n_routes, vpr, rows, dyp);
        if (c.T > 0)
            combine_bwd_kernel<false><<<(c.T + tpb - 1) / tpb, 256, 0, s>>>(dy, row_map, w, c.T, c.k, vpr, tpb, rows, dyp);
    }
    return hipGetLastError();
}

hipError_t launch_permute_bwd(const moe_config& c, const void* dxp, const int32_t* row_map, void* dx,
                              hipStream_t s) {
    if (c.T == 0) return hipSuccess;
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    const bool f32 = c.dtype == MOE_F32;
    const int vpr = c.H / (f32 ? 4 : 8);
    if (f32)
        MOE_GATHER_LAUNCH(permute_bwd_kernel, true, c.k, c.T, block_for(vpr), s, dxp, row_map, c.k, vpr, R_cap, dx);
    else
        MOE_GATHER_LAUNCH(permute_bwd_kernel, false, c.k, c.T, block_for(vpr), s, dxp, row_map, c.k, vpr, R_cap, dx);
    return hipGetLastError();
}

}  // namespace moe
