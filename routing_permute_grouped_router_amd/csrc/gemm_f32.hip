// Grouped float32 GEMMs (true fp32 arithmetic) for float32-storage layers.
//
// Same computation and device-side group handling as the bf16 path (gate/up
// projection fused with SwiGLU, then the down projection; see gemm_bf16.hip),
// on the vector ALUs with fp32 FMAs: 64-row x 64-column tiles staged through
// LDS in 16-deep K slices, each of 256 threads computing a 4 x 4 block.  In
// SwiGLU tiles the 64 B columns are 32 gate and the matching 32 up columns, and
// a thread's four columns are (gate f, gate f+1, up f, up f+1), so it forms
// silu(g) * u for its own outputs.
#include "moe_internal.h"
#include "tiles.h"

namespace moe {
namespace {

constexpr int TM = 64, TN = 64, TK = 16;

struct F32Args {
    const float* A;
    const float* B;
    const int32_t* offsets;
    int E, K, rows, n_out, b_rows;
    float* C;
    float* stash;
    // gather (gate/up only): A is x [T, K], row r of the grouped operand is
    // x[src_map[r] / gk]; the first counts[e] rows of expert e are routed, the
    // rest are padding rows (zero A rows, as in a materialised Xp)
    const int32_t* src_map;
    const int32_t* counts;
    int gk;
    const float* row_w;  // optional: output row r scaled by row_w[r] before it is stored
    float lim;           // SwiGLU clamp limit (+inf: none)
};

template <bool SWIGLU>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(F32Args p, int n_tiles) {
    __shared__ float As[TK][TM + 4];
    __shared__ float Bs[TK][TN + 4];
    __shared__ int32_t pre[kMaxExperts + 1];
    __shared__ int scan_tmp[4];
    const int tid = threadIdx.x;
    const int total_m = build_tile_prefix(p.offsets, p.E, TM, pre, scan_tmp);
    const int t = blockIdx.x;
    const int mt = t / n_tiles, nt = t % n_tiles;
    if (mt >= total_m) return;
    const int e = find_expert(pre, p.E, mt);
    const int row_end = min(p.offsets[e + 1], p.rows);
    const int row0 = p.offsets[e] + (mt - pre[e]) * TM;
    if (row0 < 0 || row0 >= row_end) return;  // only for inconsistent offsets
    const float* Be = p.B + (size_t)e * p.b_rows * p.K;
    const int ty = tid >> 4, tx = tid & 15;

    // load mapping: one float4 of A and one of B per thread per K slice
    const int lr = tid >> 2, lk = (tid & 3) * 4;
    const int a_row = row0 + lr;
    const int a_end = p.src_map ? min(p.offsets[e] + p.counts[e], row_end) : row_end;
    const float* const a_src =
        a_row < a_end ? (p.src_map ? p.A + (size_t)(p.src_map[a_row] / p.gk) * p.K : p.A + (size_t)a_row * p.K)
                      : nullptr;
    int b_row;
    if (SWIGLU) b_row = lr < 32 ? nt * 32 + lr : p.n_out + nt * 32 + (lr - 32);
    else b_row = nt * TN + lr;

    float acc[4][4] = {};
    for (int k0 = 0; k0 < p.K; k0 += TK) {
        const float4 av = a_src ? *(const float4*)(a_src + k0 + lk) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 bv = *(const float4*)(Be + (size_t)b_row * p.K + k0 + lk);
        As[lk + 0][lr] = av.x;
        As[lk + 1][lr] = av.y;
        As[lk + 2][lr] = av.z;
        As[lk + 3][lr] = av.w;
        Bs[lk + 0][lr] = bv.x;
        Bs[lk + 1][lr] = bv.y;
        Bs[lk + 2][lr] = bv.z;
        Bs[lk + 3][lr] = bv.w;
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
            if (SWIGLU) {
                b[0] = Bs[kk][tx * 2];
                b[1] = Bs[kk][tx * 2 + 1];
                b[2] = Bs[kk][32 + tx * 2];
                b[3] = Bs[kk][32 + tx * 2 + 1];
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = row0 + ty * 4 + i;
        if (r >= row_end) continue;
        const float rw = p.row_w ? p.row_w[r] : 1.f;
        if (SWIGLU) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int f = nt * 32 + tx * 2 + j;
                const float g = acc[i][j], u = acc[i][2 + j];
                const float gc = p.lim < INFINITY ? fminf(g, p.lim) : g;
                const float uc = p.lim < INFINITY ? fminf(fmaxf(u, -p.lim), p.lim) : u;
                p.C[(size_t)r * p.n_out + f] = (gc / (1.0f + expf(-gc))) * uc * rw;
                if (p.stash) {
                    p.stash[(size_t)r * 2 * p.n_out + f] = g;
                    p.stash[(size_t)r * 2 * p.n_out + p.n_out + f] = u;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) p.C[(size_t)r * p.n_out + nt * TN + tx * 4 + j] = acc[i][j] * rw;
        }
    }
}

}  // namespace

hipError_t launch_swiglu_gemm_f32(const moe_config& c, const float* xp, const float* w1, const int32_t* offsets,
                                  float* h, float* stash, const int32_t* src_map, const int32_t* counts,
                                  const float* row_w, hipStream_t s) {
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    const int n_tiles = c.F / 32;
    const int64_t blocks = (R_cap / TM + c.E) * n_tiles;
    if (blocks == 0) return hipSuccess;
    F32Args a{xp, w1, offsets, c.E, c.H, (int)R_cap, c.F, 2 * c.F, h, stash, src_map, counts, c.k, row_w,
              c.swiglu_limit > 0.f ? c.swiglu_limit : INFINITY};
    grouped_gemm_f32_kernel<true><<<(unsigned)blocks, 256, 0, s>>>(a, n_tiles);
    return hipGetLastError();
}

hipError_t launch_down_gemm_f32(const moe_config& c, const float* h, const float* w2, const int32_t* offsets,
                                float* yp, const float* row_w, hipStream_t s) {
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    const int n_tiles = c.H / TN;
    const int64_t blocks = (R_cap / TM + c.E) * n_tiles;
    if (blocks == 0) return hipSuccess;
    F32Args a{h, w2, offsets, c.E, c.F, (int)R_cap, c.H, c.H, yp, nullptr, nullptr, nullptr, 1, row_w, INFINITY};
    grouped_gemm_f32_kernel<false><<<(unsigned)blocks, 256, 0, s>>>(a, n_tiles);
    return hipGetLastError();
}

}  // namespace moe
