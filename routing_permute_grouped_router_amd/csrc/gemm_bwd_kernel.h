// Grouped bf16 GEMMs of the expert FFN backward (CDNA4, v_mfma_f32_32x32x16_bf16).
//
// The backward of the TransformerEngine page "[JAX] Expert Parallelism: JAX
// primitives + VJPs" (commit "plumb token_counts to grouped_gemm and zero
// 0-token wgrad slices": weight gradients of experts that received no rows are
// zero) and of the cudnn-frontend page "Add MoE + expert-parallel Python API
// surface, PyTorch reference, and tests" (Summary: SwiGLU recomputed from the
// saved pre-activation stash).  Three shapes, all C = A * B with float32
// accumulation:
//
//   DGRAD   C[r, n] = sum_k A[r, k] * B_e[k, n]      rows r of expert e (ragged M)
//           A row-major [rows][K] (K contiguous), B_e row-major [K][N]
//           (N contiguous: the stored weight read along its other axis);
//           epilogue: store bf16, or the SwiGLU backward with the stash.
//   WGRAD   C_e[m, n] = sum_{r of e} A[r, m] * B[r, n] (ragged K), float32 out;
//           both operands row-major over the rows r.
//
// Tiles are 256 x 256 x 64 on 4 wavefronts of 128 x 128 (4 x 4 MFMA 32x32
// accumulators), two LDS stages of 64 KiB with the same XOR-swizzled
// K-contiguous layout as the forward kernel.  Operands go global -> registers
// -> LDS: the next stage's loads are in flight during the current stage's
// MFMAs.  A K-contiguous operand is copied in 16-byte chunks; a K-strided one
// is loaded as 8 x 8 bf16 blocks (eight 16-byte rows along the contiguous
// axis) and transposed in registers so that LDS again holds 8 consecutive K
// values per 16 bytes.  Out-of-range rows and columns load zeros.
#pragma once

#include "gemm_bf16_kernel.h"

namespace moe {
namespace gemm {

enum BwdMode { kDgrad = 0, kDgradDswiglu = 1, kWgrad = 2 };

struct BwdArgs {
    const uint16_t* A;      // DGRAD: [rows][K]; WGRAD: [rows][M]
    const uint16_t* B;      // DGRAD: [E][K][N]; WGRAD: [rows][N]
    const int32_t* offsets; // [E+1]
    int E;
    int rows;               // rows allocated in the row-indexed buffers (R_cap)
    int M;                  // WGRAD: output rows per expert
    int N;                  // output columns
    int K;                  // DGRAD: contraction length
    uint16_t* C;            // DGRAD: [rows][N] bf16 (kDgrad) / [rows][2N] bf16 (kDgradDswiglu: dG | dU)
    float* Cw;              // WGRAD: [E][M][N] float32
    const uint16_t* stash;  // kDgradDswiglu: [rows][2N] bf16 (g | u)
    // WGRAD work split: an expert's rows are cut into units of at most S rows;
    // the partial sums of experts with two or more units go to workspace slots
    // [slots][M][N] (summed in unit order by wgrad_reduce_kernel), and block 0
    // records each expert's (units, first slot) in meta[E].
    float* part;
    int2* meta;
    int S;
    int slots;
};

// 8 x 8 bf16 transpose: in[i] holds row i (8 values along the contiguous axis);
// out[j] holds column j (the 8 row values, row 0 lowest).
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
    uint32_t w[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        w[i][0] = in[i].x;
        w[i][1] = in[i].y;
        w[i][2] = in[i].z;
        w[i][3] = in[i].w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t x = w[2 * p][j >> 1], y = w[2 * p + 1][j >> 1];
            o[p] = (j & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
        }
        out[j] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// Epilogue of 16 consecutive output columns n..n+15 of row r (values v).
template <int MODE>
__device__ __forceinline__ void bwd_store16(const BwdArgs& p, const float (&v)[16], float* cw, int r, int n,
                                            int row_end) {
    if (n >= p.N) return;
    if (MODE == kWgrad) {
        if (r >= p.M) return;
        float4* dst = (float4*)(cw + (size_t)r * p.N + n);
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
        return;
    }
    if (r >= row_end) return;
    if (MODE == kDgrad) {
        uint4* dst = (uint4*)(p.C + (size_t)r * p.N + n);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            dst[j] = make_uint4(pack_bf16x2(v[8 * j], v[8 * j + 1]), pack_bf16x2(v[8 * j + 2], v[8 * j + 3]),
                                pack_bf16x2(v[8 * j + 4], v[8 * j + 5]), pack_bf16x2(v[8 * j + 6], v[8 * j + 7]));
        return;
    }
    // SwiGLU backward: v = dH[r, n..]; g, u from the bf16 stash
    const uint4* gs = (const uint4*)(p.stash + (size_t)r * 2 * p.N + n);
    const uint4* us = (const uint4*)(p.stash + (size_t)r * 2 * p.N + p.N + n);
    uint4* dg = (uint4*)(p.C + (size_t)r * 2 * p.N + n);
    uint4* du = (uint4*)(p.C + (size_t)r * 2 * p.N + p.N + n);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint4 gq = gs[j], uq = us[j];
        const uint32_t gw[4] = {gq.x, gq.y, gq.z, gq.w}, uw[4] = {uq.x, uq.y, uq.z, uq.w};
        uint32_t og[4], ou[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float rg[2], ru[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float g = __uint_as_float(h ? (gw[w] & 0xffff0000u) : (gw[w] << 16));
                const float u = __uint_as_float(h ? (uw[w] & 0xffff0000u) : (uw[w] << 16));
                const float dh = v[8 * j + 2 * w + h];
                const float sg = 1.0f / (1.0f + __expf(-g));
                rg[h] = dh * u * sg * (1.0f + g * (1.0f - sg));
                ru[h] = dh * g * sg;
            }
            og[w] = pack_bf16x2(rg[0], rg[1]);
            ou[w] = pack_bf16x2(ru[0], ru[1]);
        }
        dg[j] = make_uint4(og[0], og[1], og[2], og[3]);
        du[j] = make_uint4(ou[0], ou[1], ou[2], ou[3]);
    }
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bwd(BwdArgs p) {
    constexpr int BK = 64;
    constexpr bool WG = MODE == kWgrad;
    constexpr int STAGE = kTile * BK;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[2][2][STAGE];
    __shared__ int32_t pre[kMaxExperts + 1];
    __shared__ int32_t spre[WG ? kMaxExperts + 1 : 1];
    __shared__ int scan_tmp[kThreads / 64];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int n_tiles = (p.N + kTile - 1) / kTile;
    int total, m_tiles = 0;
    if (WG) {
        // every expert owns at least one unit: empty ones write zeros
        m_tiles = (p.M + kTile - 1) / kTile;
        total = build_unit_prefix(p.offsets, p.E, p.S, pre, spre, scan_tmp) * m_tiles * n_tiles;
        if (blockIdx.x == 0)
            for (int e = tid; e < p.E; e += kThreads) p.meta[e] = make_int2(pre[e + 1] - pre[e], spre[e]);
    } else {
        total = build_tile_prefix(p.offsets, p.E, kTile, pre, scan_tmp) * n_tiles;
    }
    const int xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds;
    const int lb = blockIdx.x / kXcds;
    // Row-indexed GEMMs: every tile costs the same, so each XCD takes a
    // contiguous range.  Weight gradients: units differ in rows (hot experts
    // come first in expert order), so units are dealt to the XCDs round robin
    // (unit u to XCD u % 8) and each XCD walks the tiles of its own units.
    int t_begin, t_end;
    if (WG) {
        const int units = total / (m_tiles * n_tiles);
        t_begin = 0;
        t_end = (units > xcd ? (units - xcd + kXcds - 1) / kXcds : 0) * m_tiles * n_tiles;
    } else {
        t_begin = (int)((int64_t)total * xcd / kXcds);
        t_end = (int)((int64_t)total * (xcd + 1) / kXcds);
    }

    int arow[4], brow[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) arow[mi] = wm * 128 + mi * 32 + (lane & 31);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) brow[ni] = wn * 128 + ni * 32 + (lane & 31);

    // strided-operand loader: thread -> 8 x 8 block (k block tid / 32, column block tid % 32)
    const int sb_k = tid >> 5, sb_c = tid & 31;
    // contiguous-operand loader: 8 chunks of 16 B per thread, chunk q = tid + 256 i
    for (int t = t_begin + lb; t < t_end; t += per_xcd) {
        int e, m0, n0, k_begin, k_end, row0 = 0, row_end = 0;
        float* cw = nullptr;
        if (WG) {
            const int j = t / (m_tiles * n_tiles);
            const int rem = t - j * m_tiles * n_tiles;
            const int u = xcd + kXcds * j;
            e = find_expert(pre, p.E, u);
            const int s = u - pre[e], units = pre[e + 1] - pre[e];
            m0 = (rem / n_tiles) * kTile;
            n0 = (rem % n_tiles) * kTile;
            const int r_begin = max(0, p.offsets[e]), r_end = min(p.offsets[e + 1], p.rows);
            k_begin = min(r_begin + s * p.S, r_end);
            k_end = min(k_begin + p.S, r_end);
            if (units == 1) {
                cw = p.Cw + (size_t)e * p.M * p.N;
            } else {
                const int slot = spre[e] + s;
                if (slot >= p.slots) continue;  // only for inconsistent offsets
                cw = p.part + (size_t)slot * p.M * p.N;
            }
        } else {
            int mt, nt;
            tile_coords(t, total / n_tiles, n_tiles, 4, &mt, &nt);
            e = find_expert(pre, p.E, mt);
            row_end = min(p.offsets[e + 1], p.rows);
            row0 = p.offsets[e] + (mt - pre[e]) * kTile;
            if (row0 < 0 || row0 >= row_end) continue;  // only for inconsistent offsets
            m0 = row0;
            n0 = nt * kTile;
            k_begin = 0;
            k_end = p.K;
        }
        const int nk = k_end > k_begin ? (k_end - k_begin + BK - 1) / BK : 0;
        const uint16_t* Be = WG ? p.B : p.B + (size_t)e * p.K * p.N;
        const int a_cols = WG ? p.M : 0;

        uint4 ra[8], rb[8];
        // global -> registers for K step kt
#define GB_LOAD(kt)                                                                                       \
    {                                                                                                     \
        const int k0 = k_begin + (kt) * BK;                                                               \
        if (WG) {                                                                                         \
            _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                               \
                const int k = k0 + sb_k * 8 + i, m = m0 + sb_c * 8;                                       \
                ra[i] = (k < k_end && m < a_cols) ? *(const uint4*)(p.A + (size_t)k * a_cols + m)         \
                                                  : make_uint4(0, 0, 0, 0);                               \
            }                                                                                             \
        } else {                                                                                          \
            _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                               \
                const int q = tid + 256 * i, r = q >> 3, c = q & 7;                                       \
                const int row = m0 + r;                                                                   \
                ra[i] = row < row_end ? *(const uint4*)(p.A + (size_t)row * p.K + k0 + c * 8)             \
                                      : make_uint4(0, 0, 0, 0);                                           \
            }                                                                                             \
        }                                                                                                 \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                                   \
            const int k = k0 + sb_k * 8 + i, n = n0 + sb_c * 8;                                           \
            rb[i] = (k < k_end && n < p.N) ? *(const uint4*)(Be + (size_t)k * p.N + n)                    \
                                           : make_uint4(0, 0, 0, 0);                                      \
        }                                                                                                 \
    }
        // registers -> LDS stage st (K-contiguous swizzled rows)
#define GB_STORE(st)                                                                                      \
    {                                                                                                     \
        uint4 tr[8];                                                                                      \
        if (WG) {                                                                                         \
            transpose8x8(ra, tr);                                                                         \
            _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                               \
                const int r = sb_c * 8 + j;                                                               \
                *(uint4*)&lds[st][0][r * BK + ((sb_k ^ swz<0>(r)) << 3)] = tr[j];                         \
            }                                                                                             \
        } else {                                                                                          \
            _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                               \
                const int q = tid + 256 * i, r = q >> 3, c = q & 7;                                       \
                *(uint4*)&lds[st][0][r * BK + ((c ^ swz<0>(r)) << 3)] = ra[i];                            \
            }                                                                                             \
        }                                                                                                 \
        transpose8x8(rb, tr);                                                                             \
        _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                                   \
            const int r = sb_c * 8 + j;                                                                   \
            *(uint4*)&lds[st][1][r * BK + ((sb_k ^ swz<0>(r)) << 3)] = tr[j];                             \
        }                                                                                                 \
    }

        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

        if (nk > 0) {
            GB_LOAD(0);
            GB_STORE(0);
            __syncthreads();
        }
        for (int kt = 0; kt < nk; ++kt) {
            const int st = kt & 1;
            if (kt + 1 < nk) GB_LOAD(kt + 1);
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                const int c = kk * 2 + (lane >> 5);
                bf16x8 fa[4], fb[4];
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
                    fa[mi] = __builtin_bit_cast(
                        bf16x8, *(const uint4*)&lds[st][0][arow[mi] * BK + ((c ^ swz<0>(arow[mi])) << 3)]);
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    fb[ni] = __builtin_bit_cast(
                        bf16x8, *(const uint4*)&lds[st][1][brow[ni] * BK + ((c ^ swz<0>(brow[ni])) << 3)]);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
            }
            if (kt + 1 < nk) GB_STORE(st ^ 1);
            __syncthreads();
        }

#undef GB_LOAD
#undef GB_STORE
        // epilogue: each 32x32 accumulator goes through this wave's 4 KiB of LDS
        // (row stride 33 floats) and comes back as 16 consecutive columns of
        // one row per lane, for 32/64-byte stores.  The stage buffers are free:
        // the K loop ended with a barrier.
        float* wbuf = (float*)&lds[0][0][0] + wid * (32 * 33 + 32);
        const int rr = lane >> 1, c0 = (lane & 1) * 16;
#define GB_EPI(MI, NI)                                                                                   \
    {                                                                                                    \
        _Pragma("unroll") for (int q = 0; q < 16; ++q)                                                  \
            wbuf[(8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)) * 33 + (lane & 31)] = acc[MI][NI][q];        \
        __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0): the wave's writes are in LDS */              \
        float v[16];                                                                                     \
        _Pragma("unroll") for (int j = 0; j < 16; ++j) v[j] = wbuf[rr * 33 + c0 + j];                    \
        __builtin_amdgcn_s_waitcnt(0xC07F); /* reads done before the next tile overwrites */            \
        bwd_store16<MODE>(p, v, cw, m0 + wm * 128 + (MI) * 32 + rr, n0 + wn * 128 + (NI) * 32 + c0, row_end); \
    }
        GB_EPI(0, 0) GB_EPI(0, 1) GB_EPI(0, 2) GB_EPI(0, 3)
        GB_EPI(1, 0) GB_EPI(1, 1) GB_EPI(1, 2) GB_EPI(1, 3)
        GB_EPI(2, 0) GB_EPI(2, 1) GB_EPI(2, 2) GB_EPI(2, 3)
        GB_EPI(3, 0) GB_EPI(3, 1) GB_EPI(3, 2) GB_EPI(3, 3)
#undef GB_EPI
        __syncthreads();  // LDS reused by the next tile's loads
    }
}

}  // namespace gemm
}  // namespace moe
