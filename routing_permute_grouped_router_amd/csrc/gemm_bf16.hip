// Grouped bf16 GEMMs on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Forward of the expert FFN: the gate/up projection fused with SwiGLU and the
// down projection, per the Diagram of the TransformerEngine page "[Draft][JAX]
// MoE block optimization" (fused grouped GEMM and SwiGLU, then the down
// projection) and the cudnn-frontend page "Add MoE + expert-parallel Python
// API surface, PyTorch reference, and tests" (silu(gate) * up).  Group sizes
// come from the device `offsets` buffer, as the TransformerEngine page "[JAX]
// Expert Parallelism: JAX primitives + VJPs" does with its device token counts
// (commit "plumb token_counts to grouped_gemm ..."); empty experts own no
// tiles and ragged tails are masked.
//
// C[r, n] = sum_k A[r, k] * B_e[n, k]: both operands have K contiguous (rows of
// Xp or h, and the stored weights), so every global load is a 16-byte vector
// and every MFMA operand is one 16-byte LDS read.
//
// Block: 256 threads = 4 wavefronts in a 2 x 2 grid, tile BM x BN x BK =
// 128 x 128 x 64, each wavefront a 64 x 64 sub-tile of 2 x 2 MFMA 32x32
// accumulators.  LDS holds two stages of A and B (64 KiB); 16-byte chunks of a
// 128-byte LDS row are XOR-swizzled by (row & 7) so the MFMA operand reads of
// 32 consecutive rows spread over all banks.  Global loads of stage k+1 are in
// flight while stage k feeds the matrix cores; one barrier per K step.
//
// SwiGLU tiles take 64 gate rows (f0..f0+63) and the matching 64 up rows
// (F+f0..) of W1 into one 128-row B tile; each wavefront's two N accumulators
// are then gate and up of the same 32 columns in the same lanes, so the
// epilogue forms silu(g) * u in registers.
//
// The grid is persistent (2 blocks per CU); block b works on XCD b % 8 and the
// tile sequence is split into 8 contiguous ranges, one per XCD, walked in a
// grouped order so co-resident blocks of an XCD share A and B in its L2.
#include <algorithm>

#include "moe_internal.h"
#include "tiles.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

struct GemmArgs {
    const uint16_t* A;      // [rows, K]
    const uint16_t* B;      // [E][n_rows_per_expert][K]
    const int32_t* offsets; // [E+1]
    int E, K;
    int rows;               // rows allocated in A and C (R_cap): no access beyond
    int n_out;              // output columns (F for SwiGLU, H for down)
    int b_rows;             // rows of B per expert (2F or H)
    uint16_t* C;            // [rows, n_out]
    uint16_t* stash;        // SwiGLU only: [rows, 2F] or null
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

template <bool SWIGLU>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_bf16_kernel(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t lds_b[2][BN * BK];
    __shared__ int32_t pre[kMaxExperts + 1];
    __shared__ int scan_tmp[kThreads / 64];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int total_m = build_tile_prefix(p.offsets, p.E, BM, pre, scan_tmp);
    const int cols_per_tile = SWIGLU ? BN / 2 : BN;
    const int n_tiles = p.n_out / cols_per_tile;
    const int total = total_m * n_tiles;

    // XCD-contiguous split of the tile sequence
    const int xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds;
    const int lb = blockIdx.x / kXcds;
    const int t_begin = (int)((int64_t)total * xcd / kXcds), t_end = (int)((int64_t)total * (xcd + 1) / kXcds);

    const int K = p.K;
    const int nk = K / BK;
    // global-load mapping: 4 chunks of 16 B per operand per thread
    const int ld_row = tid >> 3, ld_chunk = tid & 7;

    for (int t = t_begin + lb; t < t_end; t += per_xcd) {
        int mt, nt;
        tile_coords(t, total_m, n_tiles, kGroupM, &mt, &nt);
        const int e = find_expert(pre, p.E, mt);
        const int row_end = min(p.offsets[e + 1], p.rows);
        const int row0 = p.offsets[e] + (mt - pre[e]) * BM;
        if (row0 < 0 || row0 >= row_end) continue;  // only for inconsistent offsets
        const uint16_t* Be = p.B + (size_t)e * p.b_rows * K;

        // per-thread source rows of the A and B tiles: chunk i covers tile row
        // ld_row + 32 i (named registers, no arrays, so nothing lands in scratch)
#define SRC(i)                                                                                   \
    const int r##i = ld_row + 32 * i;                                                            \
    const bool aok##i = row0 + r##i < row_end;                                                   \
    const uint16_t* asrc##i = p.A + (size_t)(aok##i ? row0 + r##i : 0) * K + ld_chunk * 8;       \
    const int brow##i = SWIGLU ? ((r##i < 64) ? nt * 64 + r##i : p.n_out + nt * 64 + (r##i - 64)) \
                               : nt * BN + r##i;                                                 \
    const uint16_t* bsrc##i = Be + (size_t)brow##i * K + ld_chunk * 8;                           \
    uint4 ra##i, rb##i;
        SRC(0) SRC(1) SRC(2) SRC(3)
#undef SRC
#define LD1(i, kt)                                                       \
    ra##i = *(const uint4*)(asrc##i + (kt) * BK);                        \
    if (!aok##i) ra##i = make_uint4(0, 0, 0, 0);                         \
    rb##i = *(const uint4*)(bsrc##i + (kt) * BK);
#define ST1(i, buf)                                                      \
    *(uint4*)(&lds_a[buf][swz(r##i, ld_chunk)]) = ra##i;                 \
    *(uint4*)(&lds_b[buf][swz(r##i, ld_chunk)]) = rb##i;
#define GLOAD(kt) LD1(0, kt) LD1(1, kt) LD1(2, kt) LD1(3, kt)
#define SSTORE(buf) ST1(0, buf) ST1(1, buf) ST1(2, buf) ST1(3, buf)

        f32x16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

        GLOAD(0);
        SSTORE(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int buf = kt & 1;
            if (kt + 1 < nk) { GLOAD(kt + 1); }
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                const int chunk = kk * 2 + (lane >> 5);
                bf16x8 af[2], bfr[2];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) {
                    const int r = wm * 64 + mi * 32 + (lane & 31);
                    const uint4 v = *(const uint4*)(&lds_a[buf][swz(r, chunk)]);
                    af[mi] = __builtin_bit_cast(bf16x8, v);
                }
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const int r = SWIGLU ? ni * 64 + wn * 32 + (lane & 31) : wn * 64 + ni * 32 + (lane & 31);
                    const uint4 v = *(const uint4*)(&lds_b[buf][swz(r, chunk)]);
                    bfr[ni] = __builtin_bit_cast(bf16x8, v);
                }
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
            }
            if (kt + 1 < nk) { SSTORE(buf ^ 1); }
            __syncthreads();
        }

        // epilogue: lane holds column (lane & 31) and rows 8*(q/4) + 4*(lane/32) + q%4
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int r = row0 + wm * 64 + mi * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                if (r >= row_end) continue;
                if (SWIGLU) {
                    const int f = nt * 64 + wn * 32 + (lane & 31);
                    const float g = acc[mi][0][q], u = acc[mi][1][q];
                    p.C[(size_t)r * p.n_out + f] = f32_to_bf16(silu(g) * u);
                    if (p.stash) {
                        p.stash[(size_t)r * 2 * p.n_out + f] = f32_to_bf16(g);
                        p.stash[(size_t)r * 2 * p.n_out + p.n_out + f] = f32_to_bf16(u);
                    }
                } else {
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        const int n = nt * BN + wn * 64 + ni * 32 + (lane & 31);
                        p.C[(size_t)r * p.n_out + n] = f32_to_bf16(acc[mi][ni][q]);
                    }
                }
            }
        }
    }
#undef GLOAD
#undef SSTORE
#undef LD1
#undef ST1
}

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

int persistent_grid(int64_t max_tiles) {
    int g = num_cus() * 2;
    g = (g / kXcds) * kXcds;
    if (g < kXcds) g = kXcds;
    const int64_t need = ((max_tiles + kXcds - 1) / kXcds) * kXcds;
    return (int)std::min<int64_t>(g, std::max<int64_t>(need, kXcds));
}

}  // namespace

hipError_t launch_swiglu_gemm_bf16(const moe_config& c, const uint16_t* xp, const uint16_t* w1,
                                   const int32_t* offsets, uint16_t* h, uint16_t* stash, hipStream_t s) {
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    const int64_t max_tiles = (R_cap / BM + c.E) * (c.F / (BN / 2));
    if (max_tiles == 0) return hipSuccess;
    GemmArgs a{xp, w1, offsets, c.E, c.H, (int)R_cap, c.F, 2 * c.F, h, stash};
    grouped_gemm_bf16_kernel<true><<<persistent_grid(max_tiles), kThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_down_gemm_bf16(const moe_config& c, const uint16_t* h, const uint16_t* w2, const int32_t* offsets,
                                 uint16_t* yp, hipStream_t s) {
    const int64_t R_cap = (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1);
    const int64_t max_tiles = (R_cap / BM + c.E) * (c.H / BN);
    if (max_tiles == 0) return hipSuccess;
    GemmArgs a{h, w2, offsets, c.E, c.F, (int)R_cap, c.H, c.H, yp, nullptr};
    grouped_gemm_bf16_kernel<false><<<persistent_grid(max_tiles), kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
