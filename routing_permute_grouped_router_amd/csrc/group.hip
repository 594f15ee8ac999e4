// Grouping and permutation into expert-major rows, with no host sync.
//
// The layout is the one the TransformerEngine page "[JAX] Expert Parallelism:
// JAX primitives + VJPs" describes for its dispatch output (commit "plumb
// token_counts to grouped_gemm and zero 0-token wgrad slices"): expert blocks
// back to back, each zero-padded to the alignment, per-expert counts kept in a
// device buffer that the grouped GEMMs read as their group sizes.  The tracking
// issue "MoE training optimization" asks that every problem size come from
// device buffers; here counts, offsets and maps never leave the GPU.
//
// Two launches, and no atomics decide a row: per-chunk expert histograms,
// then one fused kernel whose blocks each derive the aligned offsets and
// their chunk's bases from the histograms, rank their routes from LDS bitmaps
// (a route's rank = routes to the same expert from earlier tokens of the
// chunk, a token choosing an expert at most once) and copy their tokens' rows
// to the k destination rows with 16-byte vector accesses.
#include <algorithm>

#include "moe_internal.h"
#include "tiles.h"

namespace moe {
namespace {

constexpr int kSub = 256;         // tokens per counting chunk = threads per block
constexpr int kMaxPartRoutes = 2048;  // routes whose rows one block of the fused kernel keeps in LDS
constexpr int kNv = 16;               // row vectors a thread of the fused kernel holds at once
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // a 16-byte row vector (kept in registers)

// A route (t, j) to expert e is live when e is in [0, E) and no earlier slot
// of the same token names e (top-k never repeats an expert; a repeated id in a
// caller's table is dropped and counted as an error).
__device__ __forceinline__ bool route_ok(const int32_t* tok, int j, int32_t e, int E) {
    if (e < 0 || e >= E) return false;
    for (int q = 0; q < j; ++q)
        if (tok[q] == e) return false;
    return true;
}

// Routes per expert of each 256-token chunk: chunk_counts[c][e].
__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                    int32_t* __restrict__ chunk_counts, int32_t* __restrict__ err) {
    __shared__ int32_t cnt[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int t = blockIdx.x * kSub + threadIdx.x;
    int bad = 0;
    if (t < T) {
        for (int j = 0; j < k; ++j) {
            const int32_t e = idx[(int64_t)t * k + j];
            if (e == -1) continue;
            if (route_ok(idx + (int64_t)t * k, j, e, E)) atomicAdd(&cnt[e], 1);
            else ++bad;
        }
    }
    if (bad && err) atomicAdd(err, bad);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

struct GroupArgs {
    const int32_t* idx;
    int T, E, k, align;
    int64_t R_cap;
    const int32_t* chunk_counts;  // [n_chunks][E]
    int n_chunks, parts;          // blocks per chunk: parts, each with 256 / parts tokens
    int32_t* counts;
    int32_t* offsets;
    int32_t* row_map;
    int32_t* src_map;
    const void* x;                // [T, vpr] vectors, or null (grouping only)
    void* xp;                     // [R_cap, vpr]
    int vpr;
    const uint32_t* xs;           // MX scale rows as 4-byte words [T, svpr], or null
    uint32_t* xps;
    int svpr;
};

// The grouping and the permutation in one pass over the chunks.  Block b
// handles part b % parts of chunk b / parts:
//  1. From the chunk counts it forms every expert's total, the aligned
//     exclusive scan of the totals (the offsets) and the first row of its
//     chunk's routes of each expert (offset + routes of earlier chunks).
//     Every block does this itself, so no single-block scan sits between the
//     counting and the copy.  Block 0 also writes counts, offsets and the -1
//     src_map entries of padding rows and of the unused tail.
//  2. A 256-bit LDS bitmap per expert marks the chunk's tokens routed to it; a
//     route's rank among the chunk's routes to its expert (token order) is a
//     popcount, so its row is deterministic.  The block writes row_map and
//     src_map for the routes of its part and keeps their rows in LDS.
//  3. It copies its tokens' rows (and MXFP8 scale rows) to their k
//     destination rows, vector by vector, and zeroes the padding rows of the
//     experts e with e % gridDim == b.
template <typename V>
__global__ __launch_bounds__(256) void group_scatter_kernel(GroupArgs a) {
    extern __shared__ int32_t sm[];
    __shared__ int scan_tmp[256 / 64];
    const int E = a.E, k = a.k, tid = threadIdx.x;
    const int TP = kSub / a.parts;
    uint32_t* bits = (uint32_t*)sm;        // [E][8]
    int32_t* s_off = sm + E * 8;           // [E + 1]
    int32_t* s_base = s_off + E + 1;       // [E]
    int32_t* s_cnt = s_base + E;           // [E]
    int32_t* s_rows = s_cnt + E;           // [TP * k]
    const int c = blockIdx.x / a.parts, part = blockIdx.x % a.parts;
    const int t0 = c * kSub;
    const int ntok = max(0, min(TP, a.T - (t0 + part * TP)));
    const int64_t tbase = (int64_t)t0 + part * TP;

    // 0. The part's token rows do not depend on the maps: their first kNv
    //    vectors per thread are loaded before the grouping, which then runs
    //    while they are in flight.
    const V* __restrict__ xv = (const V*)a.x;
    V* __restrict__ xpv = (V*)a.xp;
    const int nvec = a.xp ? ntok * a.vpr : 0;
    V v[kNv];
#pragma unroll
    for (int u = 0; u < kNv; ++u) {
        const int q = tid + u * 256;
        if (q < nvec) v[u] = xv[(tbase + q / a.vpr) * a.vpr + q % a.vpr];
    }

    // 1. totals, offsets and this chunk's bases.  The chunk counts are summed
    //    by all threads (coalesced loads, eight in flight per thread, LDS
    //    atomics); then thread tid owns experts [tid * per, tid * per + per)
    //    for the aligned scan.
    for (int e = tid; e < E; e += 256) {
        s_cnt[e] = 0;
        s_base[e] = 0;
    }
    __syncthreads();
    {
        const int n = a.n_chunks * E;
        for (int q0 = tid; q0 < n; q0 += 8 * 256) {
            int w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int q = q0 + u * 256;
                w[u] = q < n ? a.chunk_counts[q] : 0;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int q = q0 + u * 256;
                if (q < n && w[u]) {
                    const int e = q % E;
                    atomicAdd(&s_cnt[e], w[u]);
                    if (q / E < c) atomicAdd(&s_base[e], w[u]);
                }
            }
        }
    }
    __syncthreads();
    const int per = (E + 255) / 256;  // <= 4
    int padded = 0;
    for (int i = 0; i < per; ++i) {
        const int e = tid * per + i;
        if (e < E) padded += (s_cnt[e] + a.align - 1) / a.align * a.align;
    }
    int total;
    int run = block_exclusive_scan(padded, scan_tmp, &total);
    for (int i = 0; i < per; ++i) {
        const int e = tid * per + i;
        if (e < E) {
            s_off[e] = run;
            s_base[e] += run;  // first row of this chunk's routes to e
            run += (s_cnt[e] + a.align - 1) / a.align * a.align;
        }
    }
    if (tid == 0) s_off[E] = total;
    for (int i = tid; i < E * 8; i += 256) bits[i] = 0;
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int e = tid; e < E; e += 256) {
            a.counts[e] = s_cnt[e];
            a.offsets[e] = s_off[e];
            for (int r = s_off[e] + s_cnt[e]; r < s_off[e + 1] && r < a.R_cap; ++r) a.src_map[r] = -1;  // padding
        }
        if (tid == 0) a.offsets[E] = total;
        for (int64_t r = total + tid; r < a.R_cap; r += 256) a.src_map[r] = -1;  // tail
    }

    // 2. ranks
    {
        const int t = t0 + tid;
        if (t < a.T) {
            const int32_t* tok = a.idx + (int64_t)t * k;
            for (int j = 0; j < k; ++j) {
                const int32_t e = tok[j];
                if (route_ok(tok, j, e, E)) atomicOr(&bits[e * 8 + (tid >> 5)], 1u << (tid & 31));
            }
        }
    }
    __syncthreads();
    for (int q = tid; q < TP * k; q += 256) {
        const int tl = part * TP + q / k, j = q % k;
        const int t = t0 + tl;
        int32_t row = -1;
        if (t < a.T) {
            const int64_t i = (int64_t)t * k + j;
            const int32_t* tok = a.idx + (int64_t)t * k;
            const int32_t e = tok[j];
            if (route_ok(tok, j, e, E)) {
                const int w = tl >> 5;
                int rank = __popc(bits[e * 8 + w] & ((1u << (tl & 31)) - 1u));
                for (int u = 0; u < w; ++u) rank += __popc(bits[e * 8 + u]);
                row = s_base[e] + rank;
                if (row < 0 || row >= a.R_cap) row = -1;  // only for inconsistent counts
                if (row >= 0) a.src_map[row] = (int32_t)i;
            }
            a.row_map[i] = row;
        }
        s_rows[q] = row;
    }
    if (!a.xp) return;
    __syncthreads();

    // 3. the part's rows to their routes' rows: the vectors loaded in step 0,
    //    then (rows longer than kNv vectors per thread) the rest in batches
    auto store_batch = [&](int q0, const V (&w)[kNv]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kNv; ++u) {
            const int q = q0 + tid + u * 256;
            if (q < nvec) {
                const int tl = q / a.vpr, col = q % a.vpr;
                for (int j = 0; j < k; ++j) {
                    const int32_t row = s_rows[tl * k + j];
                    if (row >= 0) xpv[(int64_t)row * a.vpr + col] = w[u];
                }
            }
        }
    };
    store_batch(0, v);
    for (int q0 = kNv * 256; q0 < nvec; q0 += kNv * 256) {
        V w[kNv];
#pragma unroll
        for (int u = 0; u < kNv; ++u) {
            const int q = q0 + tid + u * 256;
            if (q < nvec) w[u] = xv[(tbase + q / a.vpr) * a.vpr + q % a.vpr];
        }
        store_batch(q0, w);
    }
    if (a.xs) {
        const int n = ntok * a.svpr;
        for (int q = tid; q < n; q += 256) {
            const int tl = q / a.svpr, col = q % a.svpr;
            const uint32_t v = a.xs[(tbase + tl) * a.svpr + col];
            for (int j = 0; j < k; ++j) {
                const int32_t row = s_rows[tl * k + j];
                if (row >= 0) a.xps[(int64_t)row * a.svpr + col] = v;
            }
        }
    }
    // padding rows of Xp (and of its scales) are zero
    if (a.align > 1) {
        for (int e = blockIdx.x; e < E; e += gridDim.x) {
            const int64_t r0 = s_off[e] + s_cnt[e], r1 = min((int64_t)s_off[e + 1], a.R_cap);
            V* __restrict__ xpv = (V*)a.xp;
            const V z{};
            for (int64_t q = tid; q < (r1 - r0) * a.vpr; q += 256) xpv[r0 * a.vpr + q] = z;
            if (a.xps)
                for (int64_t q = tid; q < (r1 - r0) * a.svpr; q += 256) a.xps[r0 * a.svpr + q] = 0u;
        }
    }
}

template <typename V>
hipError_t launch_typed(GroupArgs a, hipStream_t s) {
    const size_t lds = ((size_t)a.E * 8 + (a.E + 1) + 3 * (size_t)a.E + (size_t)(kSub / a.parts) * a.k) * 4;
    group_scatter_kernel<V><<<a.n_chunks * a.parts, 256, lds, s>>>(a);
    return hipGetLastError();
}

}  // namespace

int group_n_chunks(int T, int /*E*/) { return T > 0 ? (T + kSub - 1) / kSub : 1; }

hipError_t launch_group(const moe_config& c, const int32_t* idx, const void* x, const uint8_t* x_scale, void* xp,
                        uint8_t* xp_scale, int32_t* counts, int32_t* offsets, int32_t* row_map, int32_t* src_map,
                        int32_t* err, int32_t* ws, hipStream_t s) {
    const int nch = group_n_chunks(c.T, c.E);
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    count_kernel<<<nch, 256, 0, s>>>(idx, c.T, c.E, c.k, ws, err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    GroupArgs a{idx, c.T, c.E, c.k, c.align, R_cap, ws, nch, 1, counts, offsets, row_map, src_map,
                nullptr, nullptr, 0, nullptr, nullptr, 0};
    // Parts per chunk: enough blocks to stream the copy (about 1024), and few
    // enough routes per block to keep their rows in LDS.
    int parts = 1;
    const int64_t esz = c.dtype == MOE_F32 ? 4 : (c.dtype == MOE_BF16 ? 2 : 1);
    const int64_t row_bytes = c.dtype == MOE_MXFP4 ? (int64_t)c.H / 2 : (int64_t)c.H * esz;  // MXFP4: 2 per byte
    const int64_t vec_bytes = row_bytes % 16 == 0 ? 16 : (row_bytes % 4 == 0 ? 4 : 1);
    if (xp) {
        while (parts < kSub && nch * parts < 1024) parts *= 2;
        while (parts < kSub && (kSub / parts) * (row_bytes / vec_bytes) > (int64_t)kNv * 256) parts *= 2;
    }
    while (parts < kSub && (kSub / parts) * c.k > kMaxPartRoutes) parts *= 2;
    a.parts = parts;
    if (!xp || c.T == 0) {
        a.xp = xp;  // null: grouping only; T = 0: only the padding rows (none exist) and the maps' tail
        return launch_typed<u32x4>(a, s);
    }
    a.x = x;
    a.xp = xp;
    if (c.dtype == MOE_MXFP8 || c.dtype == MOE_MXFP4) {  // H % 128 == 0: scale rows are whole 4-byte words
        a.xs = (const uint32_t*)x_scale;
        a.xps = (uint32_t*)xp_scale;
        a.svpr = c.H / kMxBlock / 4;
    }
    if (row_bytes % 16 == 0) {
        a.vpr = (int)(row_bytes / 16);
        return launch_typed<u32x4>(a, s);
    }
    if (row_bytes % 4 == 0) {
        a.vpr = (int)(row_bytes / 4);
        return launch_typed<uint32_t>(a, s);
    }
    a.vpr = (int)row_bytes;
    return launch_typed<uint8_t>(a, s);
}

}  // namespace moe
