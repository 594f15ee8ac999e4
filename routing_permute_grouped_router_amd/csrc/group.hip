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
// Three small kernels build the maps deterministically (no atomics decide a
// row): per-chunk expert histograms, one block that scans them into per-chunk
// bases and the aligned offsets, then per-chunk ranks from LDS bitmaps
// (a route's rank = routes to the same expert from earlier tokens of the chunk,
// a token choosing an expert at most once).  A fourth, bandwidth-bound kernel
// reads every token row once and writes it to its k destination rows with
// 16-byte vector accesses.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kSub = 256;          // tokens per sub-chunk = threads per block
constexpr int kMaxChunks = 128;    // chunks the scan handles
constexpr int kScanLds = 14336;    // int32 chunk counts the scan keeps in LDS (56 KiB + 4 KiB scratch)

// A route (t, j) to expert e is live when e is in [0, E) and no earlier slot
// of the same token names e (top-k never repeats an expert; a repeated id in a
// caller's table is dropped and counted as an error).
__device__ __forceinline__ bool route_ok(const int32_t* tok, int j, int32_t e, int E) {
    if (e < 0 || e >= E) return false;
    for (int q = 0; q < j; ++q)
        if (tok[q] == e) return false;
    return true;
}

__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                    int chunk_tokens, int32_t* __restrict__ chunk_counts,
                                                    int32_t* __restrict__ err) {
    __shared__ int32_t cnt[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int t0 = blockIdx.x * chunk_tokens;
    const int t1 = min(T, t0 + chunk_tokens);
    int bad = 0;
    for (int t = t0 + threadIdx.x; t < t1; t += blockDim.x) {
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

// One block of 1024 threads.  chunk_counts [n_chunks][E] becomes the exclusive
// per-expert base of each chunk (in place); counts, offsets and the -1 entries
// of src_map for padding rows and the tail are written.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ chunk_counts, int n_chunks, int E,
                                                    int align, int64_t R_cap, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets, int32_t* __restrict__ src_map) {
    extern __shared__ int32_t lds[];  // [n_chunks * E] chunk counts, then [1024] scan scratch
    int32_t* cc = lds;
    int32_t* tmp = lds + n_chunks * E;
    const int n = n_chunks * E;
    for (int i = threadIdx.x; i < n; i += blockDim.x) cc[i] = chunk_counts[i];
    __syncthreads();
    int padded = 0, total = 0;
    const int e = threadIdx.x;
    if (e < E) {
        for (int c = 0; c < n_chunks; ++c) {
            const int v = cc[c * E + e];
            cc[c * E + e] = total;
            total += v;
        }
        padded = ((total + align - 1) / align) * align;
    }
    // block-wide inclusive scan of padded (Hillis-Steele over 1024 entries)
    tmp[threadIdx.x] = padded;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int add = threadIdx.x >= off ? tmp[threadIdx.x - off] : 0;
        __syncthreads();
        tmp[threadIdx.x] += add;
        __syncthreads();
    }
    const int incl = tmp[threadIdx.x];
    const int excl = incl - padded;
    if (e < E) {
        counts[e] = total;
        offsets[e] = excl;
        for (int r = excl + total; r < incl && r < R_cap; ++r) src_map[r] = -1;  // padding rows
    }
    if (e == E - 1) offsets[E] = incl;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) chunk_counts[i] = cc[i];
    const int64_t used = tmp[E - 1];
    for (int64_t r = used + threadIdx.x; r < R_cap; r += blockDim.x) src_map[r] = -1;  // tail
}

// One block per chunk: rank of each route among the chunk's routes to the same
// expert, in token order, from 256-bit-per-expert LDS bitmaps of each
// sub-chunk of 256 tokens.
__global__ __launch_bounds__(256) void maps_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                   int chunk_tokens, int64_t R_cap,
                                                   const int32_t* __restrict__ chunk_base,
                                                   const int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ row_map, int32_t* __restrict__ src_map) {
    extern __shared__ uint32_t smem[];
    uint32_t* bits = smem;                        // [E][8] words
    int32_t* base = (int32_t*)(smem + E * 8);     // [E]
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 256) base[e] = offsets[e] + chunk_base[(int64_t)blockIdx.x * E + e];
    const int t_chunk = blockIdx.x * chunk_tokens;
    const int t_end = min(T, t_chunk + chunk_tokens);
    for (int ts = t_chunk; ts < t_end; ts += kSub) {
        for (int i = tid; i < E * 8; i += 256) bits[i] = 0;
        __syncthreads();
        const int t = ts + tid;
        const bool live = t < t_end;
        if (live) {
            for (int j = 0; j < k; ++j) {
                const int32_t e = idx[(int64_t)t * k + j];
                if (route_ok(idx + (int64_t)t * k, j, e, E)) atomicOr(&bits[e * 8 + (tid >> 5)], 1u << (tid & 31));
            }
        }
        __syncthreads();
        if (live) {
            const int word = tid >> 5;
            const uint32_t below = (1u << (tid & 31)) - 1u;
            for (int j = 0; j < k; ++j) {
                const int64_t i = (int64_t)t * k + j;
                const int32_t e = idx[i];
                if (!route_ok(idx + (int64_t)t * k, j, e, E)) {
                    row_map[i] = -1;
                    continue;
                }
                int rank = __popc(bits[e * 8 + word] & below);
                for (int q = 0; q < word; ++q) rank += __popc(bits[e * 8 + q]);
                const int32_t row = base[e] + rank;
                const bool ok = row >= 0 && row < R_cap;  // always true for consistent counts
                row_map[i] = ok ? row : -1;
                if (ok) src_map[row] = (int32_t)i;
            }
        }
        __syncthreads();
        for (int e = tid; e < E; e += 256) {
            int add = 0;
            for (int q = 0; q < 8; ++q) add += __popc(bits[e * 8 + q]);
            base[e] += add;
        }
        __syncthreads();
    }
}

// Row copy: token t's row (row_bytes bytes, a multiple of VEC) to its routes.
// Each block handles `tpb` tokens; threads stride over (token, vector) pairs.
template <typename V>
__global__ __launch_bounds__(256) void scatter_rows_kernel(const V* __restrict__ x, const int32_t* __restrict__ row_map,
                                                           int T, int k, int vec_per_row, int tpb,
                                                           int64_t n_rows, V* __restrict__ xp) {
    const int t0 = blockIdx.x * tpb;
    const int n = min(tpb, T - t0) * vec_per_row;
    for (int q = threadIdx.x; q < n; q += blockDim.x) {
        const int t = t0 + q / vec_per_row;
        const int c = q % vec_per_row;
        const V v = x[(int64_t)t * vec_per_row + c];
        for (int j = 0; j < k; ++j) {
            const int32_t r = row_map[(int64_t)t * k + j];
            if (r >= 0 && r < n_rows) xp[(int64_t)r * vec_per_row + c] = v;
        }
    }
}

// Zero the padding rows [offsets[e] + counts[e], offsets[e+1]) of expert e.
template <typename V>
__global__ __launch_bounds__(256) void zero_pad_rows_kernel(const int32_t* __restrict__ counts,
                                                            const int32_t* __restrict__ offsets, int vec_per_row,
                                                            int64_t n_rows, V* __restrict__ xp) {
    const int e = blockIdx.x;
    const int64_t r0 = max((int64_t)0, (int64_t)offsets[e] + counts[e]);
    const int64_t r1 = min((int64_t)offsets[e + 1], n_rows);
    const int64_t n = (r1 - r0) * vec_per_row;
    const V z{};
    for (int64_t q = threadIdx.x; q < n; q += blockDim.x) xp[r0 * vec_per_row + q] = z;
}

template <typename V>
hipError_t scatter_typed(const void* x, const int32_t* row_map, int T, int k, int64_t row_bytes, int64_t n_rows,
                         void* xp, hipStream_t s) {
    const int vpr = (int)(row_bytes / sizeof(V));
    const int tpb = vpr >= 256 ? 1 : (256 + vpr - 1) / vpr;
    const int grid = (T + tpb - 1) / tpb;
    scatter_rows_kernel<V><<<grid, 256, 0, s>>>((const V*)x, row_map, T, k, vpr, tpb, n_rows, (V*)xp);
    return hipGetLastError();
}

template <typename V>
hipError_t zero_pad_typed(const int32_t* counts, const int32_t* offsets, int E, int64_t row_bytes, int64_t n_rows,
                          void* xp, hipStream_t s) {
    zero_pad_rows_kernel<V><<<E, 256, 0, s>>>(counts, offsets, (int)(row_bytes / sizeof(V)), n_rows, (V*)xp);
    return hipGetLastError();
}

hipError_t scatter_any(const void* x, const int32_t* row_map, int T, int k, int64_t row_bytes, int64_t n_rows,
                       void* xp, hipStream_t s) {
    if (row_bytes % 16 == 0) return scatter_typed<uint4>(x, row_map, T, k, row_bytes, n_rows, xp, s);
    if (row_bytes % 4 == 0) return scatter_typed<uint32_t>(x, row_map, T, k, row_bytes, n_rows, xp, s);
    return scatter_typed<uint8_t>(x, row_map, T, k, row_bytes, n_rows, xp, s);
}

hipError_t zero_pad_any(const int32_t* counts, const int32_t* offsets, int E, int64_t row_bytes, int64_t n_rows,
                        void* xp, hipStream_t s) {
    if (row_bytes % 16 == 0) return zero_pad_typed<uint4>(counts, offsets, E, row_bytes, n_rows, xp, s);
    if (row_bytes % 4 == 0) return zero_pad_typed<uint32_t>(counts, offsets, E, row_bytes, n_rows, xp, s);
    return zero_pad_typed<uint8_t>(counts, offsets, E, row_bytes, n_rows, xp, s);
}

}  // namespace

int group_n_chunks(int T, int E) {
    const int max_chunks = std::min(kMaxChunks, kScanLds / E);
    const int subs = (T + kSub - 1) / kSub;                  // sub-chunks of 256 tokens
    const int per_chunk = (subs + max_chunks - 1) / max_chunks;  // sub-chunks per chunk
    const int n = per_chunk ? (subs + per_chunk - 1) / per_chunk : 0;
    return n < 1 ? 1 : n;
}

int group_chunk_tokens(int T, int E) {
    const int max_chunks = std::min(kMaxChunks, kScanLds / E);
    const int subs = (T + kSub - 1) / kSub;
    int per_chunk = (subs + max_chunks - 1) / max_chunks;
    if (per_chunk < 1) per_chunk = 1;
    return per_chunk * kSub;
}

hipError_t launch_group(const moe_config& c, const int32_t* idx, int32_t* counts, int32_t* offsets,
                        int32_t* row_map, int32_t* src_map, int32_t* err, int32_t* ws, hipStream_t s) {
    const int nch = group_n_chunks(c.T, c.E);
    const int ct = group_chunk_tokens(c.T, c.E);
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    count_kernel<<<nch, 256, 0, s>>>(idx, c.T, c.E, c.k, ct, ws, err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t scan_lds = ((size_t)nch * c.E + 1024) * sizeof(int32_t);
    scan_kernel<<<1, 1024, scan_lds, s>>>(ws, nch, c.E, c.align, R_cap, counts, offsets, src_map);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (c.T == 0) return hipSuccess;
    const size_t maps_lds = (size_t)c.E * 8 * sizeof(uint32_t) + (size_t)c.E * sizeof(int32_t);
    maps_kernel<<<nch, 256, maps_lds, s>>>(idx, c.T, c.E, c.k, ct, R_cap, ws, offsets, row_map, src_map);
    return hipGetLastError();
}

hipError_t launch_permute_rows(const moe_config& c, const void* x, const uint8_t* x_scale, const int32_t* row_map,
                               const int32_t* counts, const int32_t* offsets, void* xp, uint8_t* xp_scale,
                               hipStream_t s) {
    const int64_t esz = c.dtype == MOE_F32 ? 4 : (c.dtype == MOE_BF16 ? 2 : 1);
    const int64_t row_bytes = (int64_t)c.H * esz;
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    hipError_t e = hipSuccess;
    if (c.T > 0) {
        e = scatter_any(x, row_map, c.T, c.k, row_bytes, R_cap, xp, s);
        if (e != hipSuccess) return e;
        if (c.dtype == MOE_MXFP8) {
            e = scatter_any(x_scale, row_map, c.T, c.k, c.H / kMxBlock, R_cap, xp_scale, s);
            if (e != hipSuccess) return e;
        }
    }
    if (c.align > 1) {
        e = zero_pad_any(counts, offsets, c.E, row_bytes, R_cap, xp, s);
        if (e != hipSuccess) return e;
        if (c.dtype == MOE_MXFP8) e = zero_pad_any(counts, offsets, c.E, c.H / kMxBlock, R_cap, xp_scale, s);
    }
    return e;
}

}  // namespace moe
