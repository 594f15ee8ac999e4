// Device-side tile scheduling over ragged expert groups.
//
// Group sizes are read from `offsets` in device memory (the sync-free rule of
// the tracking issue "MoE training optimization"): every block derives the
// per-expert M-tile counts itself, so no host ever sees a count.  Experts with
// no rows own no tiles.
#pragma once

#include "moe_internal.h"

namespace moe {

// Exclusive block-wide scan of one int per thread; blockDim.x % 64 == 0.
// lds_tmp must hold blockDim.x / 64 ints.  Returns the exclusive prefix and
// writes the block total to *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds_tmp, int* total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) lds_tmp[wid] = x;
    __syncthreads();
    int base = 0, tot = 0;
    for (int q = 0; q < nw; ++q) {
        const int s = lds_tmp[q];
        base += q < wid ? s : 0;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

// pre[e] = sum_{e'<e} ceil(rows(e') / BM) for e in [0, E]; returns pre[E].
// rows(e) = offsets[e+1] - offsets[e] (padding rows included).
__device__ __forceinline__ int build_tile_prefix(const int32_t* __restrict__ offsets, int E, int BM, int32_t* pre,
                                                 int* lds_tmp) {
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int e0 = threadIdx.x * per, e1 = min(E, e0 + per);
    int local = 0;
    for (int e = e0; e < e1; ++e) local += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
    int total;
    int run = block_exclusive_scan(local, lds_tmp, &total);
    for (int e = e0; e < e1; ++e) {
        pre[e] = run;
        run += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
    }
    if (threadIdx.x == 0) pre[E] = total;
    __syncthreads();
    return total;
}

// Work units of the weight-gradient GEMMs (ragged contraction over each
// expert's rows).  An expert with rows(e) rows is cut into
// units(e) = max(1, ceil(rows(e) / S)) row ranges of at most S rows; an
// expert with no rows keeps one unit (it writes zeros).  pre[e] = sum of units
// of the experts before e; slot[e] = the same sum restricted to experts with
// two or more units (their partial sums take workspace slots).  Returns pre[E];
// slot[E] is the number of slots used.
__device__ __forceinline__ int build_unit_prefix(const int32_t* __restrict__ offsets, int E, int S, int32_t* pre,
                                                 int32_t* slot, int* lds_tmp) {
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int e0 = threadIdx.x * per, e1 = min(E, e0 + per);
    int lu = 0, ls = 0;
    for (int e = e0; e < e1; ++e) {
        const int rows = offsets[e + 1] - offsets[e];
        const int u = rows > 0 ? (rows + S - 1) / S : 1;
        lu += u;
        ls += u >= 2 ? u : 0;
    }
    int total_u, total_s;
    int run_u = block_exclusive_scan(lu, lds_tmp, &total_u);
    int run_s = block_exclusive_scan(ls, lds_tmp, &total_s);
    for (int e = e0; e < e1; ++e) {
        pre[e] = run_u;
        slot[e] = run_s;
        const int rows = offsets[e + 1] - offsets[e];
        const int u = rows > 0 ? (rows + S - 1) / S : 1;
        run_u += u;
        run_s += u >= 2 ? u : 0;
    }
    if (threadIdx.x == 0) {
        pre[E] = total_u;
        slot[E] = total_s;
    }
    __syncthreads();
    return total_u;
}

// Largest e with pre[e] <= mt (that expert is non-empty and owns M-tile mt).
__device__ __forceinline__ int find_expert(const int32_t* pre, int E, int mt) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= mt) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Tile t of a grouped GEMM: its expert e, M-tile mt (global index) and
// N-tile nt.  GM > 0: runs of GM consecutive M-tiles sweep all N-tiles, so
// blocks running together share both A rows and B columns in L2.  GM == 0:
// expert by expert, and within an expert N-tile by N-tile with the expert's
// M-tiles adjacent, so the blocks running together cover few experts and each
// weight panel is streamed from HBM once per expert.
__device__ __forceinline__ void tile_of(int t, const int32_t* pre, int E, int total_m, int n_tiles, int GM, int* e,
                                        int* mt, int* nt);
// Grouped launch order: runs of GM consecutive M-tiles sweep all N-tiles, so
// blocks running together share both A rows and B columns in L2.
__device__ __forceinline__ void tile_coords(int t, int total_m, int n_tiles, int GM, int* mt, int* nt) {
    const int sr = t / (GM * n_tiles);
    const int rem = t - sr * GM * n_tiles;
    const int gm = min(GM, total_m - sr * GM);
    *nt = rem / gm;
    *mt = sr * GM + rem % gm;
}

__device__ __forceinline__ void tile_of(int t, const int32_t* pre, int E, int total_m, int n_tiles, int GM, int* e,
                                        int* mt, int* nt) {
    if (GM > 0) {
        tile_coords(t, total_m, n_tiles, GM, mt, nt);
        *e = find_expert(pre, E, *mt);
    } else {
        const int x = find_expert(pre, E, t / n_tiles);
        const int m_e = pre[x + 1] - pre[x], li = t - pre[x] * n_tiles;
        *e = x;
        *nt = li / m_e;
        *mt = pre[x] + li % m_e;
    }
}

}  // namespace moe
