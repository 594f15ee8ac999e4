// Launchers of the expert FFN backward GEMMs (kernel in gemm_bwd_kernel.h).
//
//   moe_grouped_down_bwd:   dGU = dSwiGLU(dYp * W2_e^T, stash)   (DGRAD + SwiGLU backward)
//                           dW2_e = dYp_e^T * h_e               (WGRAD, zero for empty experts)
//   moe_grouped_swiglu_bwd: dXp = dGU * W1_e                    (DGRAD)
//                           dW1_e = dGU_e^T * Xp_e              (WGRAD, zero for empty experts)
// bf16 storage only.
#include <algorithm>

#include "gemm_bwd_kernel.h"

namespace moe {

int gemm_persistent_grid(int64_t max_tiles);

namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t rows_cap(const moe_config& c) { return (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1); }

constexpr int64_t kPartBudget = (int64_t)1 << 30;  // bytes of partial sums a weight gradient may use

// Rows per weight-gradient work unit for an [M][N] gradient.  A unit's tiles
// should take at most half of the average work of one of the 256 CUs,
// T k / 64 stages times the M x N tiles spread over 256 CUs, so that the
// dealing can still balance them; every split expert costs a float32 partial
// sum per unit and a reduction pass, so a unit is not cut smaller than that
// (and never below 4096 rows).  The result is then doubled until the partial
// sums of all split experts fit the budget.  An expert with more than S rows
// has at most 2 rows / S units, so the experts that are split use at most
// floor(2 R_cap / S) slots.  S depends on the config only, so the workspace
// query and the launch agree.
int wgrad_split_rows(const moe_config& c, int64_t M, int64_t N) {
    const int64_t tiles = cdiv(M, gemm::kTile) * cdiv(N, gemm::kTile);
    int64_t S = std::max<int64_t>(4096, (int64_t)c.T * c.k * tiles / (2 * 256) / 64 * 64);
    while ((2 * rows_cap(c) / S) * M * N * 4 > kPartBudget) S *= 2;
    return (int)S;
}

int64_t wgrad_slots(const moe_config& c, int64_t M, int64_t N) {
    return 2 * rows_cap(c) / wgrad_split_rows(c, M, N);
}

size_t wgrad_ws_bytes(const moe_config& c, int64_t M, int64_t N) {
    // partial sums, then E (units, first slot) pairs, then 2 x 8 tile counters
    return (size_t)(wgrad_slots(c, M, N) * M * N * 4) + (size_t)c.E * sizeof(int2) + 256;
}

// The tile counters of a DGRAD launch (8) and of the WGRAD launch after it (8).
int* tile_counters(const moe_config& c, int64_t M, int64_t N, void* ws) {
    return (int*)((char*)ws + wgrad_slots(c, M, N) * M * N * 4 + (size_t)c.E * sizeof(int2));
}

// Zeroes the 16 tile counters (a kernel rather than a memset node, so the
// calls stay safe to capture in a graph).
__global__ void zero_counters_kernel(int* cnt) {
    if (threadIdx.x < 2 * gemm::kXcds) cnt[threadIdx.x] = 0;
}

// dW[e] = sum over the expert's units, in unit order, of the partial sums,
// for experts with two or more units (the others were written directly).
// Every block lists those experts (in expert order) in LDS, then the grid
// covers each listed expert's matrix in turn; a thread issues the loads of up
// to 8 units before adding them, so each lane has several loads in flight.
constexpr int kReduceBatch = 8;
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const int2* __restrict__ meta, int E,
                                                           const float4* __restrict__ part, int64_t n4, int slots,
                                                           float4* __restrict__ dw) {
    __shared__ int list[kMaxExperts];
    __shared__ int scan_tmp[256 / 64];
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int e0 = threadIdx.x * per, e1 = min(E, e0 + per);
    int mine = 0;
    for (int e = e0; e < e1; ++e) mine += meta[e].x >= 2;
    int count;
    int at = block_exclusive_scan(mine, scan_tmp, &count);
    for (int e = e0; e < e1; ++e)
        if (meta[e].x >= 2) list[at++] = e;
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int li = 0; li < count; ++li) {
        const int e = list[li];
        const int2 m = meta[e];
        if (m.y < 0 || m.y + m.x > slots) continue;  // only for inconsistent offsets
        const float4* src = part + (size_t)m.y * n4;
        float4* dst = dw + (size_t)e * n4;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
            float4 a = src[i];
            for (int u0 = 1; u0 < m.x; u0 += kReduceBatch) {
                float4 b[kReduceBatch];
#pragma unroll
                for (int j = 0; j < kReduceBatch; ++j)
                    if (u0 + j < m.x) b[j] = src[(size_t)(u0 + j) * n4 + i];
#pragma unroll
                for (int j = 0; j < kReduceBatch; ++j) {
                    if (u0 + j < m.x) {
                        a.x += b[j].x;
                        a.y += b[j].y;
                        a.z += b[j].z;
                        a.w += b[j].w;
                    }
                }
            }
            dst[i] = a;
        }
    }
}

template <int MODE>
hipError_t launch(const gemm::BwdArgs& a, int64_t max_tiles, hipStream_t s) {
    if (max_tiles <= 0) return hipSuccess;
    gemm::grouped_gemm_bwd<MODE><<<gemm_persistent_grid(max_tiles), gemm::kThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_wgrad(const moe_config& c, gemm::BwdArgs w, void* ws, hipStream_t s) {
    const int64_t M = w.M, N = w.N;
    w.sched = tile_counters(c, M, N, ws) + gemm::kXcds;
    const int64_t slots = wgrad_slots(c, M, N);
    w.S = wgrad_split_rows(c, M, N);
    w.slots = (int)slots;
    w.part = (float*)ws;
    w.meta = (int2*)((char*)ws + slots * M * N * 4);
    // units are at most R_cap / S + E
    const int64_t max_units = rows_cap(c) / w.S + c.E;
    hipError_t e = launch<gemm::kWgrad>(w, max_units * cdiv(M, gemm::kTile) * cdiv(N, gemm::kTile), s);
    if (e != hipSuccess || slots == 0) return e;
    const int64_t n4 = M * N / 4;
    const int bx = (int)std::min<int64_t>(cdiv(n4, 256), 2048);
    wgrad_reduce_kernel<<<bx, 256, 0, s>>>(w.meta, c.E, (const float4*)w.part, n4, w.slots, (float4*)w.Cw);
    return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(const moe_config& c) {
    const size_t a = wgrad_ws_bytes(c, c.H, c.F), b = wgrad_ws_bytes(c, 2 * (int64_t)c.F, c.H);
    return a > b ? a : b;
}

hipError_t launch_down_bwd(const moe_config& c, const void* dyp, const void* w2, const void* h, const void* stash,
                           const int32_t* offsets, void* dgu, float* dw2, void* ws, hipStream_t s) {
    if (c.dtype != MOE_BF16) return hipErrorNotSupported;
    const int64_t R = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    int* cnt = tile_counters(c, c.H, c.F, ws);
    zero_counters_kernel<<<1, 64, 0, s>>>(cnt);
    gemm::BwdArgs d{(const uint16_t*)dyp, (const uint16_t*)w2, offsets, c.E, (int)R, 0, c.F, c.H,
                    (uint16_t*)dgu, nullptr, (const uint16_t*)stash, nullptr, nullptr, 0, 0, cnt};
    const int64_t dgrad_tiles = (R / gemm::kTile + c.E) * cdiv(c.F, gemm::kTile);
    hipError_t e;
    if (c.swiglu_limit > 0.f) {
        d.lim = c.swiglu_limit;
        e = launch<gemm::kDgradDswigluClamp>(d, dgrad_tiles, s);
    } else {
        d.lim = INFINITY;
        e = launch<gemm::kDgradDswiglu>(d, dgrad_tiles, s);
    }
    if (e != hipSuccess) return e;
    gemm::BwdArgs w{(const uint16_t*)dyp, (const uint16_t*)h, offsets, c.E, (int)R, c.H, c.F, 0,
                    nullptr, dw2, nullptr, nullptr, nullptr, 0, 0, nullptr};
    return launch_wgrad(c, w, ws, s);
}

hipError_t launch_swiglu_bwd(const moe_config& c, const void* dgu, const void* w1, const void* xp,
                             const int32_t* offsets, void* dxp, float* dw1, void* ws, hipStream_t s) {
    if (c.dtype != MOE_BF16) return hipErrorNotSupported;
    const int64_t R = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    int* cnt = tile_counters(c, 2 * (int64_t)c.F, c.H, ws);
    zero_counters_kernel<<<1, 64, 0, s>>>(cnt);
    gemm::BwdArgs d{(const uint16_t*)dgu, (const uint16_t*)w1, offsets, c.E, (int)R, 0, c.H, 2 * c.F,
                    (uint16_t*)dxp, nullptr, nullptr, nullptr, nullptr, 0, 0, cnt};
    hipError_t e = launch<gemm::kDgrad>(d, (R / gemm::kTile + c.E) * cdiv(c.H, gemm::kTile), s);
    if (e != hipSuccess) return e;
    gemm::BwdArgs w{(const uint16_t*)dgu, (const uint16_t*)xp, offsets, c.E, (int)R, 2 * c.F, c.H, 0,
                    nullptr, dw1, nullptr, nullptr, nullptr, 0, 0, nullptr};
    return launch_wgrad(c, w, ws, s);
}

}  // namespace moe
