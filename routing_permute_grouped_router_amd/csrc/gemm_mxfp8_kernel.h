// Grouped MXFP8 GEMMs on CDNA4 scaled matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 operands, E8M0 scales per 32).
//
// Same computation, tiling, device-side group handling and direct-to-LDS
// operand streaming as the bf16 kernel (gemm_bf16_kernel.h), on the MXFP8
// block-scaled format of the cudnn-frontend page "Add MoE + expert-parallel
// Python API surface, PyTorch reference, and tests" (BlockScaledTensor, block
// 32) with OCP E4M3 elements: one LDS stage is 256 rows x 128 bytes (four
// scale blocks), the K step of one MFMA is 64 bytes (two blocks).
//
// Operand layout of the scaled MFMA (measured on gfx950): lane l holds row
// l % 32 (A) or column l % 32 (B) and the 16-byte K pieces [16 h, 16 h + 16)
// and [32 + 16 h, 32 + 16 h + 16) with h = l / 32; the E8M0 scale in byte 0 of
// lane l's scale register applies to 32-block h of that row or column.  A lane
// therefore reads 16-byte chunks c0 + h and c0 + 2 + h of its LDS row and
// passes the scale of block c0 / 2 + h.  Each lane keeps one 32-bit word of
// scales (four consecutive blocks, the whole K step) per operand row it feeds,
// loaded one K step ahead.
//
// Epilogues go through LDS (one 32 x 32 accumulator at a time per wavefront)
// so each lane finishes 16 consecutive columns of one row: the SwiGLU GEMM
// forms silu(g) * u and requantises h to MXFP8 (blocks of 32 along F; the two
// lanes of a block exchange their partial max), the down GEMM stores bf16.
#pragma once

#include "gemm_bf16_kernel.h"
#include "mxfp8.h"

namespace moe {
namespace gemm {

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct MxArgs {
    const uint8_t* A;        // [rows][K] E4M3 codes
    const uint8_t* As;       // [rows][K/32] E8M0 scales
    const uint8_t* B;        // [E][b_rows][K]
    const uint8_t* Bs;       // [E][b_rows][K/32]
    const int32_t* offsets;  // [E+1]
    int E, K, rows, n_out, b_rows;
    uint8_t* C;              // SwiGLU: h codes [rows][n_out]
    uint8_t* Cs;             // SwiGLU: h scales [rows][n_out/32]
    uint16_t* Cb;            // down: Yp bf16 [rows][n_out]
    uint16_t* stash;         // SwiGLU, optional: bf16 g | u [rows][2 n_out]
};

template <bool SWIGLU>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_mxfp8(MxArgs p) {
    constexpr int BKB = 128;               // K bytes per stage
    constexpr int CH = BKB / 16;           // 16-byte chunks per LDS row
    constexpr int RPL = 64 / CH;           // rows per wave-wide load
    constexpr int LOADS = 64 / RPL;        // loads per wave per operand per stage
    constexpr int STAGE = kTile * BKB;     // bytes of one operand stage

    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2][STAGE];
    __shared__ int32_t pre[kMaxExperts + 1];
    __shared__ int scan_tmp[kThreads / 64];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1, half = lane >> 5;
    const int total_m = build_tile_prefix(p.offsets, p.E, kTile, pre, scan_tmp);
    const int cols_per_tile = SWIGLU ? kTile / 2 : kTile;
    const int n_tiles = (p.n_out + cols_per_tile - 1) / cols_per_tile;
    const int total = total_m * n_tiles;
    const int xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds;
    const int lb = blockIdx.x / kXcds;
    const int t_begin = (int)((int64_t)total * xcd / kXcds), t_end = (int)((int64_t)total * (xcd + 1) / kXcds);

    const int K = p.K, KS = K / 32;  // bytes per row, scale bytes per row
    const int nk = K / BKB;
    const int lrow = lane / CH, lslot = lane % CH;

    int arow[4], brow[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) arow[mi] = wm * 128 + mi * 32 + (lane & 31);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
        brow[ni] = SWIGLU ? (ni < 2 ? 0 : 128) + wn * 64 + (ni & 1) * 32 + (lane & 31)
                          : wn * 128 + ni * 32 + (lane & 31);

    for (int t = t_begin + lb; t < t_end; t += per_xcd) {
        int mt, nt;
        tile_coords(t, total_m, n_tiles, 4, &mt, &nt);
        const int e = find_expert(pre, p.E, mt);
        const int row_end = min(p.offsets[e + 1], p.rows);
        const int row0 = p.offsets[e] + (mt - pre[e]) * kTile;
        if (row0 < 0 || row0 >= row_end) continue;  // only for inconsistent offsets

        auto b_row_of = [&](int r) __attribute__((always_inline)) {
            if (SWIGLU) {
                const int f = min(nt * 128 + (r & 127), p.n_out - 1);
                return r < 128 ? f : p.n_out + f;
            }
            return min(nt * kTile + r, p.n_out - 1);
        };
        uint32_t aoff[LOADS], boff[LOADS];
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int r = wid * 64 + i * RPL + lrow;
            const int chunk = lslot ^ swz<0>(r);
            aoff[i] = (uint32_t)((size_t)(min(row0 + r, row_end - 1) - row0) * K + chunk * 16);
            boff[i] = (uint32_t)((size_t)b_row_of(r) * K + chunk * 16);
        }
        const uint8_t* acodes = p.A + (size_t)row0 * K;  // A offsets are tile-relative
        const uint8_t* bcodes = p.B + (size_t)e * p.b_rows * K;
        const uint8_t* bscales = p.Bs + (size_t)e * p.b_rows * KS;
        // scale rows of this lane's MFMA operands
        const uint8_t* asr[4];
        const uint8_t* bsr[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) asr[mi] = p.As + (size_t)min(row0 + arow[mi], row_end - 1) * KS;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) bsr[ni] = bscales + (size_t)b_row_of(brow[ni]) * KS;

        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

#define GM_LOAD(kt, stage)                                                                               \
    _Pragma("unroll") for (int i = 0; i < LOADS; ++i) {                                                  \
        __builtin_amdgcn_global_load_lds((glb_void*)(acodes + aoff[i] + (size_t)(kt) * BKB),                  \
                                         (lds_void*)&lds[stage][0][(wid * 64 + i * RPL) * BKB], 16, 0, 0); \
        __builtin_amdgcn_global_load_lds((glb_void*)(bcodes + boff[i] + (size_t)(kt) * BKB),               \
                                         (lds_void*)&lds[stage][1][(wid * 64 + i * RPL) * BKB], 16, 0, 0); \
    }
#define GM_SCALES(kt, SA, SB)                                                                            \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                                      \
        SA[i] = *(const uint32_t*)(asr[i] + (kt) * 4);                                                    \
        SB[i] = *(const uint32_t*)(bsr[i] + (kt) * 4);                                                    \
    }
        uint32_t sa[4], sb[4], sa_n[4], sb_n[4];
        GM_LOAD(0, 0);
        GM_SCALES(0, sa, sb);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int st = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) {
                GM_LOAD(kt + 1, st ^ 1);
                GM_SCALES(kt + 1, sa_n, sb_n);
            }
#pragma unroll
            for (int s = 0; s < BKB / 64; ++s) {
                const int c0 = 4 * s;
                i32x8 fa[4], fb[4];
                int xa[4], xb[4];
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    const int r = arow[mi];
                    const uint4 lo = *(const uint4*)&lds[st][0][r * BKB + (((c0 + half) ^ swz<0>(r)) << 4)];
                    const uint4 hi = *(const uint4*)&lds[st][0][r * BKB + (((c0 + 2 + half) ^ swz<0>(r)) << 4)];
                    fa[mi] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    xa[mi] = (int)((sa[mi] >> (8 * (2 * s + half))) & 0xffu);
                }
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    const int r = brow[ni];
                    const uint4 lo = *(const uint4*)&lds[st][1][r * BKB + (((c0 + half) ^ swz<0>(r)) << 4)];
                    const uint4 hi = *(const uint4*)&lds[st][1][r * BKB + (((c0 + 2 + half) ^ swz<0>(r)) << 4)];
                    fb[ni] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    xb[ni] = (int)((sb[ni] >> (8 * (2 * s + half))) & 0xffu);
                }
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fa[mi], fb[ni], acc[mi][ni], 0, 0, 0, xa[mi], 0, xb[ni]);
            }
            if (more) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sa[i] = sa_n[i];
                    sb[i] = sb_n[i];
                }
            }
            __syncthreads();  // next stage landed (vmcnt 0); this stage fully read
        }
#undef GM_LOAD
#undef GM_SCALES

        // epilogue through LDS: lane -> row rr, columns c0 .. c0+15 of a 32x32 tile
        float* wb = (float*)&lds[0][0][0] + wid * 2 * (32 * 33 + 32);
        float* wb2 = wb + 32 * 33 + 32;
        const int rr = lane >> 1, cc = (lane & 1) * 16;
#define GM_STAGE_TILE(BUF, MI, NI)                                                                       \
    _Pragma("unroll") for (int q = 0; q < 16; ++q)                                                      \
        BUF[(8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)) * 33 + (lane & 31)] = acc[MI][NI][q];
        if (SWIGLU) {
#define GM_EPI_SW(MI, NI)                                                                                \
    {                                                                                                    \
        GM_STAGE_TILE(wb, MI, NI)                                                                        \
        GM_STAGE_TILE(wb2, MI, (NI) + 2)                                                                 \
        __builtin_amdgcn_s_waitcnt(0xC07F);                                                              \
        float hv[16], gv[16], uv[16];                                                                    \
        float amax = 0.f;                                                                                \
        _Pragma("unroll") for (int j = 0; j < 16; ++j) {                                                 \
            gv[j] = wb[rr * 33 + cc + j];                                                                \
            uv[j] = wb2[rr * 33 + cc + j];                                                               \
            hv[j] = silu(gv[j]) * uv[j];                                                                 \
            amax = fmaxf(amax, fabsf(hv[j]));                                                            \
        }                                                                                                \
        __builtin_amdgcn_s_waitcnt(0xC07F);                                                              \
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));                                                     \
        const int r = row0 + wm * 128 + (MI) * 32 + rr;                                                  \
        const int f = nt * 128 + wn * 64 + (NI) * 32 + cc;                                               \
        if (r < row_end && f < p.n_out) {                                                                \
            const int se = mx_shared_exp(amax);                                                          \
            uint32_t w4[4];                                                                              \
            _Pragma("unroll") for (int j = 0; j < 4; ++j)                                               \
                w4[j] = (uint32_t)e4m3_rne(ldexpf(hv[4 * j], -se)) |                                     \
                        ((uint32_t)e4m3_rne(ldexpf(hv[4 * j + 1], -se)) << 8) |                          \
                        ((uint32_t)e4m3_rne(ldexpf(hv[4 * j + 2], -se)) << 16) |                         \
                        ((uint32_t)e4m3_rne(ldexpf(hv[4 * j + 3], -se)) << 24);                          \
            *(uint4*)(p.C + (size_t)r * p.n_out + f) = make_uint4(w4[0], w4[1], w4[2], w4[3]);           \
            if ((lane & 1) == 0) p.Cs[(size_t)r * (p.n_out / 32) + f / 32] = (uint8_t)(se + 127);        \
            if (p.stash) {                                                                               \
                uint4* gs = (uint4*)(p.stash + (size_t)r * 2 * p.n_out + f);                             \
                uint4* us = (uint4*)(p.stash + (size_t)r * 2 * p.n_out + p.n_out + f);                   \
                _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                         \
                    gs[j] = make_uint4(pack_bf16x2(gv[8 * j], gv[8 * j + 1]), pack_bf16x2(gv[8 * j + 2], gv[8 * j + 3]), \
                                       pack_bf16x2(gv[8 * j + 4], gv[8 * j + 5]), pack_bf16x2(gv[8 * j + 6], gv[8 * j + 7])); \
                    us[j] = make_uint4(pack_bf16x2(uv[8 * j], uv[8 * j + 1]), pack_bf16x2(uv[8 * j + 2], uv[8 * j + 3]), \
                                       pack_bf16x2(uv[8 * j + 4], uv[8 * j + 5]), pack_bf16x2(uv[8 * j + 6], uv[8 * j + 7])); \
                }                                                                                        \
            }                                                                                            \
        }                                                                                                \
    }
            GM_EPI_SW(0, 0) GM_EPI_SW(0, 1) GM_EPI_SW(1, 0) GM_EPI_SW(1, 1)
            GM_EPI_SW(2, 0) GM_EPI_SW(2, 1) GM_EPI_SW(3, 0) GM_EPI_SW(3, 1)
#undef GM_EPI_SW
        } else {
#define GM_EPI_DN(MI, NI)                                                                                \
    {                                                                                                    \
        GM_STAGE_TILE(wb, MI, NI)                                                                        \
        __builtin_amdgcn_s_waitcnt(0xC07F);                                                              \
        float v[16];                                                                                     \
        _Pragma("unroll") for (int j = 0; j < 16; ++j) v[j] = wb[rr * 33 + cc + j];                      \
        __builtin_amdgcn_s_waitcnt(0xC07F);                                                              \
        const int r = row0 + wm * 128 + (MI) * 32 + rr;                                                  \
        const int n = nt * kTile + wn * 128 + (NI) * 32 + cc;                                            \
        if (r < row_end && n < p.n_out) {                                                                \
            uint4* dst = (uint4*)(p.Cb + (size_t)r * p.n_out + n);                                       \
            _Pragma("unroll") for (int j = 0; j < 2; ++j)                                               \
                dst[j] = make_uint4(pack_bf16x2(v[8 * j], v[8 * j + 1]), pack_bf16x2(v[8 * j + 2], v[8 * j + 3]), \
                                    pack_bf16x2(v[8 * j + 4], v[8 * j + 5]), pack_bf16x2(v[8 * j + 6], v[8 * j + 7])); \
        }                                                                                                \
    }
            GM_EPI_DN(0, 0) GM_EPI_DN(0, 1) GM_EPI_DN(0, 2) GM_EPI_DN(0, 3)
            GM_EPI_DN(1, 0) GM_EPI_DN(1, 1) GM_EPI_DN(1, 2) GM_EPI_DN(1, 3)
            GM_EPI_DN(2, 0) GM_EPI_DN(2, 1) GM_EPI_DN(2, 2) GM_EPI_DN(2, 3)
            GM_EPI_DN(3, 0) GM_EPI_DN(3, 1) GM_EPI_DN(3, 2) GM_EPI_DN(3, 3)
#undef GM_EPI_DN
        }
#undef GM_STAGE_TILE
        __syncthreads();  // LDS reused by the next tile's loads
    }
}

}  // namespace gemm
}  // namespace moe
