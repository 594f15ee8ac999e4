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

// Grouped launch order: runs of GM consecutive M-tiles sweep all N-tiles, so
// blocks running together share both A rows and B columns in L2.
__device__ __forceinline__ void tile_coords(int t, int total_m, int n_tiles, int GM, int* mt, int* nt) {
    const int sr = t / (GM * n_tiles);
    const int rem = t - sr * GM * n_tiles;
    const int gm = min(GM, total_m - sr * GM);
    *nt = rem / gm;
    *mt = sr * GM + rem % gm;
}

}  // namespace moe
