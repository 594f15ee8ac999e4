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

// Tuned on MI355X with the Mixtral-shaped and fine-grained layers (kGroupM = 0:
// tiles expert by expert, each weight panel streamed once; kSwizzle = 0: no
// LDS bank conflicts in the fragment reads, and half the LDS-active cycles of
// mode 2 at the same speed).
constexpr int kSwizzle = 0, kGroupM = 0;

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

size_t gemm_bf16_ws_bytes(const moe_config& c) {
    if (c.dtype != MOE_BF16) return 0;
    return 256 + (size_t)gemm::kXcds * gemm::kSlotsPerXcd * gemm::kTile * gemm::kTile * sizeof(float);
}

namespace {

// Zeroes the work-queue counters (a kernel rather than a memset node, so the
// calls stay safe to capture in a graph).
__global__ void zero_sched_kernel(int* sched) {
    if (threadIdx.x < gemm::kXcds) sched[threadIdx.x] = 0;
}

// Rows [32 c, 32 c + 32) of split tile j of XCD blockIdx.y (blockIdx.x =
// 8 j + c): the float32 partial sums of its S K-parts are added in part
// order, then the epilogue of the grouped GEMM is applied (SwiGLU: h =
// silu(g) * u rounded to bf16, plus the g | u stash; down: rounding to bf16).
// The queue layout is recomputed from the same offsets and block count as the
// GEMM launch.
constexpr int kReduceRows = 32;
template <bool SWIGLU, int GM>
__global__ __launch_bounds__(256) void split_reduce_bf16(gemm::Args p, int nb) {
    __shared__ int32_t pre[kMaxExperts + 1];
    __shared__ int scan_tmp[256 / 64];
    constexpr int kChunks = gemm::kTile / kReduceRows;
    const int x = blockIdx.y, j = blockIdx.x / kChunks, c = blockIdx.x % kChunks;
    const int nk = p.K / 64;
    const int total_m = build_tile_prefix(p.offsets, p.E, gemm::kTile, pre, scan_tmp);
    const int cols_per_tile = SWIGLU ? gemm::kTile / 2 : gemm::kTile;
    const int n_tiles = (p.n_out + cols_per_tile - 1) / cols_per_tile;
    const gemm::Queue q = gemm::xcd_queue(total_m * n_tiles, x, nb, nk);
    if (q.S < 2 || j >= (q.units - q.whole) / q.S) return;
    int mt, nt, e;
    tile_of(q.tb + q.whole + j, pre, p.E, total_m, n_tiles, GM, &e, &mt, &nt);
    const int row_end = min(p.offsets[e + 1], p.rows);
    const int row0 = p.offsets[e] + (mt - pre[e]) * gemm::kTile;
    if (row0 < 0 || row0 >= row_end) return;
    const int r_lo = c * kReduceRows, r_hi = min(r_lo + kReduceRows, row_end - row0);
    if (r_lo >= r_hi) return;
    // gather: rows from a_end on are padding rows, stored as zeros
    const int a_end = p.src_map ? min(p.offsets[e] + p.counts[e], row_end) : row_end;
    constexpr int kPart = gemm::kTile * gemm::kTile;
    const float* part = p.part + (size_t)(x * gemm::kSlotsPerXcd + j * q.S) * kPart;
    constexpr int kQuads = SWIGLU ? 32 : 64;  // float4 columns per row handled here
    for (int i = threadIdx.x; i < (r_hi - r_lo) * kQuads; i += blockDim.x) {
        const int r = r_lo + i / kQuads, col = (i % kQuads) * 4;
        const int n = nt * cols_per_tile + col;
        if (n >= p.n_out) continue;
        // all parts' loads first, then the sums in part order
        float4 v[gemm::kMaxSplit], w[gemm::kMaxSplit];
#pragma unroll
        for (int s = 0; s < gemm::kMaxSplit; ++s) {
            if (s < q.S) {
                v[s] = *(const float4*)(part + (size_t)s * kPart + r * gemm::kTile + col);
                if (SWIGLU) w[s] = *(const float4*)(part + (size_t)s * kPart + r * gemm::kTile + 128 + col);
            }
        }
        float4 g = v[0], u = SWIGLU ? w[0] : v[0];
#pragma unroll
        for (int s = 1; s < gemm::kMaxSplit; ++s) {
            if (s < q.S) {
                g.x += v[s].x; g.y += v[s].y; g.z += v[s].z; g.w += v[s].w;
                if (SWIGLU) { u.x += w[s].x; u.y += w[s].y; u.z += w[s].z; u.w += w[s].w; }
            }
        }
        const size_t row = (size_t)(row0 + r);
        const float rw = p.row_w ? p.row_w[row] : 1.f;
        // the SwiGLU inputs, clamped when a limit is set (the stash keeps g, u)
        float4 gc = g, uc = u;
        if (SWIGLU && p.lim < INFINITY) {
            gc.x = fminf(g.x, p.lim); gc.y = fminf(g.y, p.lim); gc.z = fminf(g.z, p.lim); gc.w = fminf(g.w, p.lim);
            uc.x = fminf(fmaxf(u.x, -p.lim), p.lim); uc.y = fminf(fmaxf(u.y, -p.lim), p.lim);
            uc.z = fminf(fmaxf(u.z, -p.lim), p.lim); uc.w = fminf(fmaxf(u.w, -p.lim), p.lim);
        }
        if (SWIGLU) {
            *(uint2*)(p.C + row * p.n_out + n) =
                row0 + r < a_end ? make_uint2(pack_bf16x2(silu(gc.x) * uc.x * rw, silu(gc.y) * uc.y * rw),
                                              pack_bf16x2(silu(gc.z) * uc.z * rw, silu(gc.w) * uc.w * rw))
                                 : make_uint2(0u, 0u);
            if (p.stash) {
                *(uint2*)(p.stash + row * 2 * p.n_out + n) = make_uint2(pack_bf16x2(g.x, g.y), pack_bf16x2(g.z, g.w));
                *(uint2*)(p.stash + row * 2 * p.n_out + p.n_out + n) =
                    make_uint2(pack_bf16x2(u.x, u.y), pack_bf16x2(u.z, u.w));
            }
        } else {
            *(uint2*)(p.C + row * p.n_out + n) =
                make_uint2(pack_bf16x2(g.x * rw, g.y * rw), pack_bf16x2(g.z * rw, g.w * rw));
        }
    }
}

template <bool SWIGLU>
hipError_t launch_bf16(gemm::Args a, int64_t max_tiles, void* ws, hipStream_t s) {
    const int grid = gemm_persistent_grid(max_tiles);
    a.sched = (int*)ws;
    a.part = (float*)((char*)ws + 256);
    zero_sched_kernel<<<1, 64, 0, s>>>(a.sched);
    // epilogue variant: row weights (bit 1), SwiGLU clamp (bit 2)
    const int ep = (a.row_w ? 1 : 0) | (SWIGLU && a.lim < INFINITY ? 2 : 0);
    if (ep == 0) gemm::grouped_gemm_bf16<SWIGLU, kSwizzle, kGroupM, 0><<<grid, gemm::kThreads, 0, s>>>(a);
    else if (ep == 1) gemm::grouped_gemm_bf16<SWIGLU, kSwizzle, kGroupM, 1><<<grid, gemm::kThreads, 0, s>>>(a);
    else if constexpr (SWIGLU) {
        if (ep == 2) gemm::grouped_gemm_bf16<SWIGLU, kSwizzle, kGroupM, 2><<<grid, gemm::kThreads, 0, s>>>(a);
        else gemm::grouped_gemm_bf16<SWIGLU, kSwizzle, kGroupM, 3><<<grid, gemm::kThreads, 0, s>>>(a);
    }
    split_reduce_bf16<SWIGLU, kGroupM><<<dim3(gemm::kSlotsPerXcd * (gemm::kTile / kReduceRows), gemm::kXcds), 256, 0, s>>>(
        a, grid / gemm::kXcds);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_swiglu_gemm_bf16(const moe_config& c, const uint16_t* xp, const uint16_t* w1,
                                   const int32_t* offsets, uint16_t* h, uint16_t* stash, const int32_t* src_map,
                                   const int32_t* counts, const float* row_w, void* ws, hipStream_t s) {
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    const int64_t max_tiles = (R_cap / gemm::kTile + c.E) * ((c.F + 127) / 128);
    if (max_tiles == 0) return hipSuccess;
    gemm::Args a{xp, w1, offsets, c.E, c.H, (int)R_cap, c.F, 2 * c.F, h, stash, nullptr, nullptr,
                 src_map, counts, c.k, row_w, c.swiglu_limit > 0.f ? c.swiglu_limit : INFINITY};
    return launch_bf16<true>(a, max_tiles, ws, s);
}

hipError_t launch_down_gemm_bf16(const moe_config& c, const uint16_t* h, const uint16_t* w2, const int32_t* offsets,
                                 uint16_t* yp, const float* row_w, void* ws, hipStream_t s) {
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    const int64_t max_tiles = (R_cap / gemm::kTile + c.E) * ((c.H + gemm::kTile - 1) / gemm::kTile);
    if (max_tiles == 0) return hipSuccess;
    gemm::Args a{h, w2, offsets, c.E, c.F, (int)R_cap, c.H, c.H, yp, nullptr, nullptr, nullptr,
                 nullptr, nullptr, 1, row_w, INFINITY};
    return launch_bf16<false>(a, max_tiles, ws, s);
}

}  // namespace moe
