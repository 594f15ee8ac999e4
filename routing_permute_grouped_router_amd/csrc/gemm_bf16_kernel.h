// Grouped bf16 GEMM kernel template for CDNA4 (v_mfma_f32_32x32x16_bf16).
//
// C[r, n] = sum_k A[r, k] * B_e[n, k] for the rows r of expert e, group sizes
// read from the device `offsets` buffer.  Both operands have K contiguous (rows
// of Xp or h, and the stored weights), so every global load is 16 bytes and
// every MFMA operand is one 16-byte LDS read.
//
// Block: 256 threads = 4 wavefronts in a 2 x 2 grid; tile 256 x 256 x 64; each
// wavefront owns a 128 x 128 sub-tile held in 4 x 4 MFMA 32x32 accumulators
// (256 accumulator registers per lane).  Operand tiles go from global memory
// straight into LDS with global_load_lds_dwordx4 (lane i of one load lands at
// LDS base + 16 i), two stages of 64 KiB, so K step k+1 streams in while step
// k feeds the matrix cores.  In LDS each row's 16-byte K chunks are XOR-
// permuted by a function of the row (swz) so that the MFMA operand reads of
// consecutive rows hit distinct banks; the permutation is applied on the global side (a lane fetches
// the chunk its LDS slot must hold).  Rows past a group's end, and columns past
// the output width, load a clamped valid row and are never stored.
//
// SwiGLU tiles put 128 gate rows (f0..f0+127) and the matching 128 up rows
// (F+f0..) of W1 in one 256-row B tile; a wavefront's accumulators (mi, ni) and
// (mi, ni+2) are then gate and up of the same outputs in the same lanes, and
// the epilogue forms silu(g) * u in registers.
//
// The grid is persistent (one block per CU); block b runs on XCD b % 8 and
// the tile sequence is cut into 8 contiguous ranges, one per XCD, walked in a
// grouped order (GM M-tiles sweep the N-tiles) so the blocks of an XCD share A
// rows and B columns in its L2.
#pragma once

#include "moe_internal.h"
#include "tiles.h"

namespace moe {
namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int kTile = 256;
constexpr int kThreads = 256;
constexpr int kXcds = 8;

struct Args {
    const uint16_t* A;      // [rows, K]
    const uint16_t* B;      // [E][b_rows][K]
    const int32_t* offsets; // [E+1]
    int E, K;
    int rows;               // rows allocated in A and C (R_cap): no access beyond
    int n_out;              // output columns (F for SwiGLU, H for down)
    int b_rows;             // rows of B per expert (2F or H)
    uint16_t* C;            // [rows, n_out]
    uint16_t* stash;        // SwiGLU only: [rows, 2F] or null
};

// XOR mask applied to a row's 16-byte K chunk index in LDS (CH chunks per
// row).  128-byte rows: mode 0 spreads any 8 consecutive rows over distinct
// banks of a 32-bank LDS, mode 1 also any 16 over a 64-bank one.  64-byte rows
// (two per 128 bytes): the same two guarantees with the row pair folded in.
template <int SWZ, int CH = 8>
__device__ __forceinline__ int swz(int row) {
    if (CH == 8) return SWZ == 1 ? ((row ^ (row >> 3)) & 7) : (row & 7);
    return SWZ == 1 ? (((row >> 1) ^ (row >> 3)) & 3) : ((row >> 1) & 3);
}

// Epilogue helpers.  GE_STAGE_TILE writes one 32 x 32 fp32 accumulator tile
// (lane = column, slot q = row 8 (q / 4) + 4 (lane / 32) + q % 4) into a
// wavefront-private LDS tile with a 33-float row pitch; GE_PACK8 packs eight
// floats of an array into bf16 (round to nearest even) as one 16-byte word.
#define GE_STAGE_TILE(BUF, ACC)                                                                          \
    _Pragma("unroll") for (int q = 0; q < 16; ++q)                                                      \
        BUF[(8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)) * 33 + (lane & 31)] = (ACC)[q];
#define GE_PACK8(V, O)                                                                                   \
    make_uint4(pack_bf16x2((V)[(O)], (V)[(O) + 1]), pack_bf16x2((V)[(O) + 2], (V)[(O) + 3]),            \
               pack_bf16x2((V)[(O) + 4], (V)[(O) + 5]), pack_bf16x2((V)[(O) + 6], (V)[(O) + 7]))

// Direct epilogue helpers.  A 32 x 32 fp32 accumulator tile holds, in lane l
// and slot q, row 8 (q / 4) + 4 (l / 32) + q % 4 of column l % 32.  pair_bf16
// rounds it to bf16 (nearest even) and regroups it with the neighbouring lane
// (l ^ 1, a DPP quad permute) so that word p of lane l holds the two adjacent
// columns (l % 32) & ~1 and +1 of row pair_row(p, l).
// An accumulator element read out of its AGPR where it is used, so the
// compiler does not copy every accumulator to VGPRs as the K loop ends.
__device__ __forceinline__ float agpr_read(float a) {
    float v;
    __asm__ volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}
__device__ __forceinline__ float swap_lane1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ int pair_row(int p, int lane) {
    return 8 * (p >> 1) + 4 * (lane >> 5) + 2 * (p & 1) + (lane & 1);
}
__device__ __forceinline__ void pair_bf16(const float (&v)[16], int lane, uint32_t (&out)[8]) {
    const bool odd = lane & 1;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const float recv = swap_lane1(odd ? v[2 * p] : v[2 * p + 1]);
        const float lo = odd ? recv : v[2 * p], hi = odd ? v[2 * p + 1] : recv;
        out[p] = pack_bf16x2(lo, hi);
    }
}

// The same regrouping without rounding: float32 pairs.
__device__ __forceinline__ void pair_f32(const float (&v)[16], int lane, float2 (&out)[8]) {
    const bool odd = lane & 1;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const float recv = swap_lane1(odd ? v[2 * p] : v[2 * p + 1]);
        out[p] = make_float2(odd ? recv : v[2 * p], odd ? v[2 * p + 1] : recv);
    }
}

template <bool SWIGLU, int SWZ, int GM, int EARLY = 0>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bf16(Args p) {
    constexpr int BK = 64;                  // K depth of one stage
    constexpr int CH = BK / 8;              // 16-byte chunks per LDS row
    constexpr int RPL = 64 / CH;            // rows per wave-wide load
    constexpr int LOADS = 64 / RPL;         // loads per wave per operand per stage
    constexpr int STAGE_ELEMS = kTile * BK; // one operand of one stage

    __shared__ __attribute__((aligned(1024))) uint16_t lds[2][2][STAGE_ELEMS];
    __shared__ int32_t pre[kMaxExperts + 1];
    __shared__ int scan_tmp[kThreads / 64];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int total_m = build_tile_prefix(p.offsets, p.E, kTile, pre, scan_tmp);
    const int cols_per_tile = SWIGLU ? kTile / 2 : kTile;
    const int n_tiles = (p.n_out + cols_per_tile - 1) / cols_per_tile;  // last N tile may be partial
    const int total = total_m * n_tiles;

    const int xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds;
    const int lb = blockIdx.x / kXcds;
    const int t_begin = (int)((int64_t)total * xcd / kXcds), t_end = (int)((int64_t)total * (xcd + 1) / kXcds);

    const int K = p.K;
    const int nk = K / BK;
    const int lrow = lane / CH, lslot = lane % CH;

    // LDS rows of this lane's MFMA operands
    int arow[4], brow[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) arow[mi] = wm * 128 + mi * 32 + (lane & 31);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
        brow[ni] = SWIGLU ? (ni < 2 ? 0 : 128) + wn * 64 + (ni & 1) * 32 + (lane & 31)
                          : wn * 128 + ni * 32 + (lane & 31);

    for (int t = t_begin + lb; t < t_end; t += per_xcd) {
        int mt, nt;
        tile_coords(t, total_m, n_tiles, GM, &mt, &nt);
        const int e = find_expert(pre, p.E, mt);
        const int row_end = min(p.offsets[e + 1], p.rows);
        const int row0 = p.offsets[e] + (mt - pre[e]) * kTile;
        if (row0 < 0 || row0 >= row_end) continue;  // only for inconsistent offsets

        // Per-lane byte offsets of the A and B loads (K offset 0) against the
        // uniform bases: 32-bit, so the loads take few registers.
        uint32_t aoff[LOADS], boff[LOADS];
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int r = wid * 64 + i * RPL + lrow;  // tile row 0..255
            const int chunk = lslot ^ swz<SWZ>(r);
            const int ar = min(row0 + r, row_end - 1);
            aoff[i] = (uint32_t)(((size_t)(ar - row0) * K + chunk * 8) * 2);
            int br;
            if (SWIGLU) {
                const int f = min(nt * 128 + (r & 127), p.n_out - 1);
                br = r < 128 ? f : p.n_out + f;
            } else {
                br = min(nt * kTile + r, p.n_out - 1);
            }
            boff[i] = (uint32_t)(((size_t)br * K + chunk * 8) * 2);
        }
        const char* abase = (const char*)(p.A + (size_t)row0 * K);  // A offsets are tile-relative
        const char* bbase = (const char*)(p.B + (size_t)e * p.b_rows * K);

        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

#define GG_LOAD_A(kt, stage, i)                                                                          \
    __builtin_amdgcn_global_load_lds((glb_void*)(abase + aoff[i] + (size_t)(kt) * (BK * 2)),              \
                                     (lds_void*)&lds[stage][0][(wid * 64 + (i) * RPL) * BK], 16, 0, 0)
#define GG_LOAD_B(kt, stage, i)                                                                          \
    __builtin_amdgcn_global_load_lds((glb_void*)(bbase + boff[i] + (size_t)(kt) * (BK * 2)),              \
                                     (lds_void*)&lds[stage][1][(wid * 64 + (i) * RPL) * BK], 16, 0, 0)
#define GG_READ(stage, kk, FA, FB)                                                                       \
    {                                                                                                    \
        const int c_ = (kk) * 2 + (lane >> 5);                                                            \
        _Pragma("unroll") for (int mi = 0; mi < 4; ++mi) FA[mi] = __builtin_bit_cast(                    \
            bf16x8, *(const uint4*)(&lds[stage][0][arow[mi] * BK + ((c_ ^ swz<SWZ>(arow[mi])) << 3)]));    \
        _Pragma("unroll") for (int ni = 0; ni < 4; ++ni) FB[ni] = __builtin_bit_cast(                    \
            bf16x8, *(const uint4*)(&lds[stage][1][brow[ni] * BK + ((c_ ^ swz<SWZ>(brow[ni])) << 3)]));    \
    }
#define GG_MFMAS(FA, FB)                                                                                 \
    _Pragma("unroll") for (int mi = 0; mi < 4; ++mi) _Pragma("unroll") for (int ni = 0; ni < 4; ++ni)    \
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[mi], FB[ni], acc[mi][ni], 0, 0, 0);
#define GG_ISSUE(kt, stage)                                                                              \
    _Pragma("unroll") for (int i = 0; i < LOADS; ++i) {                                                  \
        GG_LOAD_A(kt, stage, i);                                                                         \
        GG_LOAD_B(kt, stage, i);                                                                         \
    }

        // Two LDS stages.  Within a stage the four 16-deep K sub-steps alternate
        // two fragment register sets, so the LDS reads of sub-step j+1 and a
        // quarter of the next stage's global loads are in flight while the
        // 16 MFMAs of sub-step j run.
        bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            GG_LOAD_A(0, 0, i);
            GG_LOAD_B(0, 0, i);
        }
        __syncthreads();
        GG_READ(0, 0, fa0, fb0);
        for (int kt = 0; kt < nk; ++kt) {
            const int st = kt & 1;
            const bool more = kt + 1 < nk;
            GG_READ(st, 1, fa1, fb1);
            if (more) {
#pragma unroll
                for (int i = 0; i < LOADS / 2; ++i) GG_LOAD_A(kt + 1, st ^ 1, i);
                if (EARLY) {
#pragma unroll
                    for (int i = 0; i < LOADS / 2; ++i) GG_LOAD_B(kt + 1, st ^ 1, i);
                }
            }
            GG_MFMAS(fa0, fb0);
            GG_READ(st, 2, fa0, fb0);
            if (more) {
#pragma unroll
                for (int i = LOADS / 2; i < LOADS; ++i) GG_LOAD_A(kt + 1, st ^ 1, i);
                if (EARLY) {
#pragma unroll
                    for (int i = LOADS / 2; i < LOADS; ++i) GG_LOAD_B(kt + 1, st ^ 1, i);
                }
            }
            GG_MFMAS(fa1, fb1);
            GG_READ(st, 3, fa1, fb1);
            if (more && !EARLY) {
#pragma unroll
                for (int i = 0; i < LOADS / 2; ++i) GG_LOAD_B(kt + 1, st ^ 1, i);
            }
            GG_MFMAS(fa0, fb0);
            if (more && !EARLY) {
#pragma unroll
                for (int i = LOADS / 2; i < LOADS; ++i) GG_LOAD_B(kt + 1, st ^ 1, i);
            }
            GG_MFMAS(fa1, fb1);
            if (more) {
                __syncthreads();  // next stage landed (vmcnt 0); this stage fully read by every wave
                GG_READ(st ^ 1, 0, fa0, fb0);
            }
        }
#undef GG_LOAD_A
#undef GG_LOAD_B
#undef GG_READ
#undef GG_MFMAS
#undef GG_ISSUE
        __syncthreads();  // every wave done with both stages before the next tile's loads

        // Epilogue straight from the accumulators: each 32 x 32 tile becomes 8
        // bf16 pairs per lane (two adjacent columns of one row, one DPP lane
        // swap per pair), stored as 4-byte words; 32 lanes cover 128
        // contiguous bytes of a row.  No LDS, so no barrier before the next tile.
        // Opaque copies of the tile's first row and of the lane index: the
        // address arithmetic below then stays after the K loop (it is not
        // hoisted out of the tile loop, where it would hold registers).
        int rbase = row0, ln = lane;
        __asm__ volatile("" : "+v"(rbase), "+v"(ln));
        const int c2 = (ln & 31) & ~1;                // even column of this lane's pairs
        const int prow = 4 * (ln >> 5) + (ln & 1);    // row of this lane's pair 0 in a 32-row block
        const int rlim = row_end - rbase;  // rows of the tile that exist
        const uint32_t ldw = (uint32_t)p.n_out / 2;  // 4-byte words per output row
        // Store the 8 pairs of a 32-row block whose first row (tile-relative) is
        // RB0 from word pointer DST (this lane's pair-0 address), LDW words per
        // row; the rows are checked only when the block runs past the group's end.
#define GB_STORE_PAIRS(DST, LDW, RB0, VP)                                                                \
    if ((RB0) + 32 <= rlim) {                                                                            \
        _Pragma("unroll") for (int q = 0; q < 8; ++q)                                                    \
            (DST)[(8 * (q >> 1) + 2 * (q & 1)) * (LDW)] = (VP)[q];                                       \
    } else {                                                                                             \
        _Pragma("unroll") for (int q = 0; q < 8; ++q)                                                    \
            if ((RB0) + prow + 8 * (q >> 1) + 2 * (q & 1) < rlim)                                        \
                (DST)[(8 * (q >> 1) + 2 * (q & 1)) * (LDW)] = (VP)[q];                                   \
    }
        if (SWIGLU) {
            uint16_t* const cbase = p.C + (size_t)rbase * p.n_out;
            uint16_t* const sbase = p.stash ? p.stash + (size_t)rbase * 2 * p.n_out : nullptr;
#define GB_EPI_SW(MI, NI)                                                                                \
    {                                                                                                    \
        const int f = nt * 128 + wn * 64 + (NI) * 32 + c2;                                               \
        const int rb0 = wm * 128 + (MI) * 32;                                                            \
        float hv[16];                                                                                    \
        float gv[16], uv[16];                                                                            \
        _Pragma("unroll") for (int q = 0; q < 16; ++q) {                                                 \
            gv[q] = agpr_read(acc[MI][NI][q]);                                                           \
            uv[q] = agpr_read(acc[MI][(NI) + 2][q]);                                                     \
            hv[q] = silu(gv[q]) * uv[q];                                                                 \
        }                                                                                                \
        uint32_t hp[8];                                                                                  \
        pair_bf16(hv, lane, hp);                                                                         \
        if (f < p.n_out) {                                                                               \
            uint32_t* dst = (uint32_t*)(cbase + (uint32_t)((rb0 + prow) * p.n_out + f));                 \
            GB_STORE_PAIRS(dst, ldw, rb0, hp)                                                                 \
            if (sbase) {                                                                                 \
                uint32_t gp[8], up[8];                                                                   \
                pair_bf16(gv, lane, gp);                                                                 \
                pair_bf16(uv, lane, up);                                                                 \
                uint32_t* gd = (uint32_t*)(sbase + (uint32_t)((rb0 + prow) * 2 * p.n_out + f));          \
                GB_STORE_PAIRS(gd, 2 * ldw, rb0, gp)                                                              \
                uint32_t* ud = gd + ldw;                                                                 \
                GB_STORE_PAIRS(ud, 2 * ldw, rb0, up)                                                              \
            }                                                                                            \
        }                                                                                                \
    }                                                                                                    \
    __builtin_amdgcn_sched_barrier(0);
            GB_EPI_SW(0, 0) GB_EPI_SW(0, 1) GB_EPI_SW(1, 0) GB_EPI_SW(1, 1)
            GB_EPI_SW(2, 0) GB_EPI_SW(2, 1) GB_EPI_SW(3, 0) GB_EPI_SW(3, 1)
#undef GB_EPI_SW
        } else {
            uint16_t* const cbase = p.C + (size_t)rbase * p.n_out;
#define GB_EPI_DN(MI, NI)                                                                                \
    {                                                                                                    \
        const int n = nt * kTile + wn * 128 + (NI) * 32 + c2;                                            \
        const int rb0 = wm * 128 + (MI) * 32;                                                            \
        float v[16];                                                                                     \
        _Pragma("unroll") for (int q = 0; q < 16; ++q) v[q] = agpr_read(acc[MI][NI][q]);                 \
        uint32_t vp[8];                                                                                  \
        pair_bf16(v, lane, vp);                                                                          \
        if (n < p.n_out) {                                                                               \
            uint32_t* dst = (uint32_t*)(cbase + (uint32_t)((rb0 + prow) * p.n_out + n));                 \
            GB_STORE_PAIRS(dst, ldw, rb0, vp)                                                                 \
        }                                                                                                \
    }                                                                                                    \
    __builtin_amdgcn_sched_barrier(0);
            GB_EPI_DN(0, 0) GB_EPI_DN(0, 1) GB_EPI_DN(0, 2) GB_EPI_DN(0, 3)
            GB_EPI_DN(1, 0) GB_EPI_DN(1, 1) GB_EPI_DN(1, 2) GB_EPI_DN(1, 3)
            GB_EPI_DN(2, 0) GB_EPI_DN(2, 1) GB_EPI_DN(2, 2) GB_EPI_DN(2, 3)
            GB_EPI_DN(3, 0) GB_EPI_DN(3, 1) GB_EPI_DN(3, 2) GB_EPI_DN(3, 3)
#undef GB_EPI_DN
        }
#undef GB_STORE_PAIRS
    }
}

}  // namespace gemm
}  // namespace moe
